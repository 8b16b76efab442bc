// Device-side helpers shared by the prefill and decode kernels of
// libmamba_scan: io element conversion and the scalar nonlinearities of the
// mixer (calm-mamba 0.1.4 PKG-INFO, "Mamba operator": SiLU after the conv and
// on the gate, softplus on the step size), built on the gfx950 hardware
// exp2 / log2 / reciprocal instructions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mscan {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// io element types: 0 = float32, 1 = bfloat16 stored as its 16 raw bits.
template <int IO>
struct Io;

template <>
struct Io<0> {
  using T = float;
  static __device__ __forceinline__ float load(const T* p) { return *p; }
  static __device__ __forceinline__ float cvt(T v) { return v; }
  static __device__ __forceinline__ void store(T* p, float v) { *p = v; }
};

template <>
struct Io<1> {
  using T = uint16_t;
  // bfloat16 -> float32 is exact: the 16 bits are the high half of the float.
  static __device__ __forceinline__ float cvt(T v) { return __uint_as_float(static_cast<uint32_t>(v) << 16); }
  static __device__ __forceinline__ float load(const T* p) { return cvt(*p); }
  // float32 -> bfloat16, round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
  static __device__ __forceinline__ T from_float(float v) { return __builtin_bit_cast(uint16_t, static_cast<__bf16>(v)); }
  static __device__ __forceinline__ void store(T* p, float v) { *p = from_float(v); }
};

__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float log2_hw(float x) { return __builtin_amdgcn_logf(x); }
__device__ __forceinline__ float rcp_hw(float x) { return __builtin_amdgcn_rcpf(x); }

// SiLU(u) = u * sigmoid(u) = u / (1 + e^-u). For u -> -inf, e^-u -> inf and
// the reciprocal gives 0, so the result tends to -0 without a NaN.
__device__ __forceinline__ float silu(float u) { return u * rcp_hw(1.0f + exp2_hw(-u * kLog2e)); }

// softplus(v) = log(1 + e^v) = max(v, 0) + log1p(e^-|v|).
// log1p(e) is taken as log(w) - c with w = fl(1 + e) and c = (w - 1) - e, the
// rounding error of w (both subtractions are exact: w - 1 by Sterbenz's lemma
// for w in [1, 2], and (w - 1) - e because w - 1 lies within a factor of two
// of e, or is 0 when w rounds to 1). log(1 + e) = log(w) + log(1 - c / w), and
// replacing c / w by c errs by c * e / w, a relative error below 2^-24; when w
// rounds to 1 the result is exactly e.
__device__ __forceinline__ float softplus(float v) {
  const float e = exp2_hw(-fabsf(v) * kLog2e);
  const float w = 1.0f + e;
  const float c = (w - 1.0f) - e;
  return fmaxf(v, 0.0f) + fmaf(log2_hw(w), kLn2, -c);
}

}  // namespace mscan
