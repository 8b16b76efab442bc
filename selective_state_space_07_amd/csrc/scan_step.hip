// One-token decode kernel of libmamba_scan for gfx950 (niverel-mamba 0.1.0
// PKG-INFO, "Autoregressive decoding": the step maps (states, token) to
// (output, new states); calm-mamba 0.1.4 PKG-INFO, O(1) state-cached
// generation). The arithmetic is the prefill's with one timestep: the conv
// window is (conv_state[0..2], x), the new conv state drops the oldest entry.
//
// The step moves ~160 bytes of state per channel and does O(d_state) math,
// so it is bound by HBM bandwidth. The main kernel gives each channel
// d_state/4 lanes; lane g owns state entries 4g..4g+3, a 16-byte slice of the
// channel's state row, so a wave's state loads and stores are contiguous 1 KiB
// runs. Every lane of the group recomputes the channel's conv/softplus terms
// (cheap next to the memory traffic); the readout's partial sums are combined
// across the group with DPP lane swaps. A one-lane-per-channel kernel serves
// calls whose state or A pointers are not 16-byte aligned.
//
// Each lane reads all of its state before the wave writes any, so an output
// state array may be the input array itself.
#include "scan_device.h"
#include "scan_internal.h"

namespace mscan {

namespace {

constexpr int kBlock = 256;

// A value rounded to the io dtype and back (the value a layer that stores it
// in that dtype would read back).
template <int IO>
__device__ __forceinline__ float io_round(float v) {
  if constexpr (IO == 1) {
    return Io<1>::cvt(Io<1>::from_float(v));
  } else {
    return v;
  }
}

// The low-rank dt of the token (dt_proj inside the step): dt[b][d] =
// sum_k dt_low[b][k] w_dt[d][k] over k < rank. A lane sums the contiguous
// range [k0, k1) of k, four terms per 8- or 16-byte load where both rows are
// aligned to it (the measured layer's rows are), one at a time otherwise.
struct LowRankDt {
  const void* dtl;     // dt_low rows, `stride` io elements apart
  int32_t stride;
  const void* w;       // w_dt [d_inner][rank] io
  int32_t rank;
  int32_t zs;          // the batch rows of z are zs elements apart (a layer's in_proj output row holds x and z)
};
template <int IO>
__device__ __forceinline__ void load4(const typename Io<IO>::T* p, float (&v)[4]);
template <int IO>
__device__ __forceinline__ float lowrank_part(const LowRankDt& q, int32_t b, int32_t d, int k0, int k1) {
  using T = typename Io<IO>::T;
  const T* lr = static_cast<const T*>(q.dtl) + static_cast<int64_t>(b) * q.stride;
  const T* wr = static_cast<const T*>(q.w) + static_cast<int64_t>(d) * q.rank;
  float acc = 0.0f;
  int k = k0;
  const uintptr_t al = reinterpret_cast<uintptr_t>(lr + k) | reinterpret_cast<uintptr_t>(wr + k);
  if ((al & (4 * sizeof(T) - 1)) == 0) {
    for (; k + 4 <= k1; k += 4) {
      float lv[4], wv[4];
      load4<IO>(lr + k, lv);
      load4<IO>(wr + k, wv);
#pragma unroll
      for (int j = 0; j < 4; ++j) acc = fmaf(lv[j], wv[j], acc);
    }
  }
  for (; k < k1; ++k) acc = fmaf(Io<IO>::load(lr + k), Io<IO>::load(wr + k), acc);
  return acc;
}

// XIN: x holds the activated conv output xc of the token (the caller ran the
// conv); the conv states are neither read nor written.
// DTP (with XIN): dt is not given; it is dt_low . w_dt[d] (dt_proj), rounded
// to the io dtype as a layer storing dt would.
template <int IO, int N, bool XIN = false, bool DTP = false>
__global__ __launch_bounds__(kBlock) void scan_step_kernel(
    int32_t batch, int32_t d_inner, int32_t bcs, LowRankDt lrd, const typename Io<IO>::T* __restrict__ x,
    const typename Io<IO>::T* __restrict__ dt, const typename Io<IO>::T* __restrict__ z,
    const typename Io<IO>::T* __restrict__ Bm, const typename Io<IO>::T* __restrict__ Cm,
    const float* __restrict__ conv_w, const float* __restrict__ conv_b,
    const float* __restrict__ dt_bias, const float* __restrict__ Dskip,
    const float* __restrict__ A, const float* conv_state_in, const float* ssm_state_in,
    typename Io<IO>::T* __restrict__ y, float* conv_state_out, float* ssm_state_out) {
  // conv/ssm state in and out may be the same arrays: no __restrict__ there.
  const int64_t i = static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x;
  if (i >= static_cast<int64_t>(batch) * d_inner) return;
  const int32_t b = static_cast<int32_t>(i / d_inner);
  const int32_t d = static_cast<int32_t>(i - static_cast<int64_t>(b) * d_inner);

  const float c0 = XIN ? 0.0f : conv_state_in[i * 3 + 0];
  const float c1 = XIN ? 0.0f : conv_state_in[i * 3 + 1];
  const float c2 = XIN ? 0.0f : conv_state_in[i * 3 + 2];
  float h[N];
#pragma unroll
  for (int n = 0; n < N; ++n) h[n] = ssm_state_in[i * N + n];

  const float xv = Io<IO>::load(x + i);
  float xc = xv;
  if (!XIN) {
    float u = fmaf(conv_w[d * 4 + 0], c0, conv_b[d]);
    u = fmaf(conv_w[d * 4 + 1], c1, u);
    u = fmaf(conv_w[d * 4 + 2], c2, u);
    u = fmaf(conv_w[d * 4 + 3], xv, u);
    xc = silu(u);
  }
  const float dtv = DTP ? io_round<IO>(lowrank_part<IO>(lrd, b, d, 0, lrd.rank)) : Io<IO>::load(dt + i);
  const float delta = softplus(dtv + dt_bias[d]);
  const float dx = delta * xc;
  const typename Io<IO>::T* Bt = Bm + static_cast<int64_t>(b) * bcs;  // rows bcs elements apart
  const typename Io<IO>::T* Ct = Cm + static_cast<int64_t>(b) * bcs;
  float acc = 0.0f;
#pragma unroll
  for (int n = 0; n < N; ++n) {
    const float dA = exp2_hw(delta * (A[d * N + n] * kLog2e));
    h[n] = fmaf(dA, h[n], dx * Io<IO>::load(Bt + n));
    acc = fmaf(Io<IO>::load(Ct + n), h[n], acc);
  }
  const float out = fmaf(Dskip[d], xc, acc) * silu(Io<IO>::load(z + (DTP ? static_cast<int64_t>(b) * lrd.zs + d : i)));
  Io<IO>::store(y + i, out);

#pragma unroll
  for (int n = 0; n < N; ++n) ssm_state_out[i * N + n] = h[n];
  if (!XIN) {
    conv_state_out[i * 3 + 0] = c1;
    conv_state_out[i * 3 + 1] = c2;
    conv_state_out[i * 3 + 2] = xv;
  }
}

// Sum of v over the lanes of each group of G = 2 or 4 consecutive lanes
// (DPP quad permutations: swap neighbours, then swap pairs).
template <int G>
__device__ __forceinline__ float group_sum(float v) {
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));  // [1,0,3,2]
  if (G == 4) v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false));  // [2,3,0,1]
  return v;
}

template <int IO>
__device__ __forceinline__ void load4(const typename Io<IO>::T* p, float (&v)[4]) {
  if (IO == 0) {
    const float4 q = *reinterpret_cast<const float4*>(p);
    v[0] = q.x; v[1] = q.y; v[2] = q.z; v[3] = q.w;
  } else {
    const uint2 q = *reinterpret_cast<const uint2*>(p);
    v[0] = __uint_as_float(q.x << 16); v[1] = __uint_as_float(q.x & 0xFFFF0000u);
    v[2] = __uint_as_float(q.y << 16); v[3] = __uint_as_float(q.y & 0xFFFF0000u);
  }
}

// The states are touched once per call: their loads and stores are marked
// non-temporal so that they do not evict the parameters and B/C rows that
// every channel group re-reads from the caches.
typedef float f32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ float stream_load(const float* p) { return __builtin_nontemporal_load(p); }
__device__ __forceinline__ float4 stream_load(const float4* p) {
  const f32x4 v = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
  return make_float4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void stream_store(float v, float* p) { __builtin_nontemporal_store(v, p); }
__device__ __forceinline__ void stream_store(float4 v, float4* p) {
  const f32x4 w = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(w, reinterpret_cast<f32x4*>(p));
}

// G = N/4 lanes per channel, each owning a float4 slice of the state vector;
// the readout is summed across the group with DPP. Needs 16-byte aligned
// ssm states and A, and B/C rows (bcs elements apart) aligned to their
// 4-element loads.
template <int IO, int N, bool XIN = false, bool DTP = false>
__global__ __launch_bounds__(kBlock) void scan_step_vec_kernel(
    int32_t batch, int32_t d_inner, int32_t bcs, LowRankDt lrd, const typename Io<IO>::T* __restrict__ x,
    const typename Io<IO>::T* __restrict__ dt, const typename Io<IO>::T* __restrict__ z,
    const typename Io<IO>::T* __restrict__ Bm, const typename Io<IO>::T* __restrict__ Cm,
    const float* __restrict__ conv_w, const float* __restrict__ conv_b,
    const float* __restrict__ dt_bias, const float* __restrict__ Dskip,
    const float* __restrict__ A, const float* conv_state_in, const float* ssm_state_in,
    typename Io<IO>::T* __restrict__ y, float* conv_state_out, float* ssm_state_out) {
  constexpr int G = N / 4;
  const int32_t total = batch * d_inner;  // < 2^31 (checked by the API)
  // total * G lanes can pass 2^31 (and a dispatch dimension's 2^32): the
  // workgroups are numbered over a 2D grid and the lane index is 64-bit
  const int64_t t = (static_cast<int64_t>(blockIdx.y) * gridDim.x + blockIdx.x) * kBlock + threadIdx.x;
  const int g = static_cast<int>(threadIdx.x) % G;
  // Lanes past the end mirror the last channel so that every group stays
  // complete for the DPP reduction; they store nothing.
  const bool act = t / G < total;
  const int32_t i = act ? static_cast<int32_t>(t / G) : total - 1;
  const int32_t b = i / d_inner;
  const int32_t d = i - b * d_inner;
  const int64_t i64 = i;

  // all loads first
  const float c0 = XIN ? 0.0f : stream_load(conv_state_in + i64 * 3 + 0);
  const float c1 = XIN ? 0.0f : stream_load(conv_state_in + i64 * 3 + 1);
  const float c2 = XIN ? 0.0f : stream_load(conv_state_in + i64 * 3 + 2);
  const float4 hs = stream_load(reinterpret_cast<const float4*>(ssm_state_in + i64 * N + 4 * g));
  const float4 a4 = *reinterpret_cast<const float4*>(A + static_cast<int64_t>(d) * N + 4 * g);
  float Bv[4], Cv[4];
  load4<IO>(Bm + static_cast<int64_t>(b) * bcs + 4 * g, Bv);
  load4<IO>(Cm + static_cast<int64_t>(b) * bcs + 4 * g, Cv);
  const float xv = Io<IO>::load(x + i64);
  // with DTP the group's lanes share the dot product, lane g a contiguous quarter (half)
  float dtv;
  if (DTP) {
    const int per = (((lrd.rank + G - 1) / G) + 3) & ~3;  // a multiple of 4 terms per lane
    const int k0 = min(g * per, lrd.rank), k1 = min(k0 + per, lrd.rank);
    dtv = io_round<IO>(group_sum<G>(lowrank_part<IO>(lrd, b, d, k0, k1)));
  } else {
    dtv = Io<IO>::load(dt + i64);
  }
  const float zv = Io<IO>::load(z + (DTP ? static_cast<int64_t>(b) * lrd.zs + d : i64));

  // causal conv over (c0, c1, c2, x), then SiLU
  float xc = xv;
  if (!XIN) {
    float u = fmaf(conv_w[d * 4 + 0], c0, conv_b[d]);
    u = fmaf(conv_w[d * 4 + 1], c1, u);
    u = fmaf(conv_w[d * 4 + 2], c2, u);
    u = fmaf(conv_w[d * 4 + 3], xv, u);
    xc = silu(u);
  }
  const float delta = softplus(dtv + dt_bias[d]);
  const float dx = delta * xc;
  const float h_in[4] = {hs.x, hs.y, hs.z, hs.w};
  const float a_in[4] = {a4.x, a4.y, a4.z, a4.w};
  float h[4];
  float acc = 0.0f;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const float dA = exp2_hw(delta * (a_in[k] * kLog2e));
    h[k] = fmaf(dA, h_in[k], dx * Bv[k]);
    acc = fmaf(Cv[k], h[k], acc);
  }
  acc = group_sum<G>(acc);
  if (!act) return;
  stream_store(make_float4(h[0], h[1], h[2], h[3]), reinterpret_cast<float4*>(ssm_state_out + i64 * N + 4 * g));
  if (g == 0) Io<IO>::store(y + i64, fmaf(Dskip[d], xc, acc) * silu(zv));
  // new conv state (c1, c2, x): entry j written by lane j of the group
  if (XIN) {
  } else if (G == 4) {
    if (g < 3) stream_store(g == 0 ? c1 : (g == 1 ? c2 : xv), conv_state_out + i64 * 3 + g);
  } else if (g == 0) {
    stream_store(c1, conv_state_out + i64 * 3 + 0);
    stream_store(c2, conv_state_out + i64 * 3 + 1);
  } else {
    stream_store(xv, conv_state_out + i64 * 3 + 2);
  }
}

template <int IO, int N, bool XIN, bool DTP>
hipError_t launch_typed(const StepCall& c) {
  const LowRankDt lrd{c.dt_low, c.dtl_stride, c.w_dt, c.dt_rank, c.z_stride ? c.z_stride : c.d_inner};
  using T = typename Io<IO>::T;
  const int64_t total = static_cast<int64_t>(c.batch) * c.d_inner;
  auto al16 = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; };
  auto al8 = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 7u) == 0; };
  // every row of B and C must start at a 4-element boundary
  const bool io_al = (IO == 0 ? (al16(c.B) && al16(c.C)) : (al8(c.B) && al8(c.C))) && c.bc_stride % 4 == 0;
  if (al16(c.ssm_state_in) && al16(c.ssm_state_out) && al16(c.A) && io_al) {
    // a dispatch counts each dimension's work-items in 32 bits: at most 2^22
    // workgroups along x, the rest along y
    const int64_t blocks = (total * (N / 4) + kBlock - 1) / kBlock;
    const int64_t gx = blocks < (int64_t{1} << 22) ? blocks : (int64_t{1} << 22);
    const dim3 grid(static_cast<unsigned>(gx), static_cast<unsigned>((blocks + gx - 1) / gx));
    hipLaunchKernelGGL((scan_step_vec_kernel<IO, N, XIN, DTP>), grid, dim3(kBlock), 0, c.stream, c.batch, c.d_inner,
                       c.bc_stride, lrd,
                       static_cast<const T*>(c.x), static_cast<const T*>(c.dt), static_cast<const T*>(c.z),
                       static_cast<const T*>(c.B), static_cast<const T*>(c.C), c.conv_w, c.conv_b, c.dt_bias,
                       c.D, c.A, c.conv_state_in, c.ssm_state_in, static_cast<T*>(c.y), c.conv_state_out,
                       c.ssm_state_out);
    return hipGetLastError();
  }
  const dim3 grid(static_cast<unsigned>((total + kBlock - 1) / kBlock));
  hipLaunchKernelGGL((scan_step_kernel<IO, N, XIN, DTP>), grid, dim3(kBlock), 0, c.stream, c.batch, c.d_inner,
                     c.bc_stride, lrd,
                     static_cast<const T*>(c.x), static_cast<const T*>(c.dt), static_cast<const T*>(c.z),
                     static_cast<const T*>(c.B), static_cast<const T*>(c.C), c.conv_w, c.conv_b, c.dt_bias,
                     c.D, c.A, c.conv_state_in, c.ssm_state_in, static_cast<T*>(c.y), c.conv_state_out,
                     c.ssm_state_out);
  return hipGetLastError();
}

}  // namespace

template <bool XIN, bool DTP>
hipError_t launch_step_x(const StepCall& c) {
  if (c.io_dtype == 0) return c.d_state == 16 ? launch_typed<0, 16, XIN, DTP>(c) : launch_typed<0, 8, XIN, DTP>(c);
  return c.d_state == 16 ? launch_typed<1, 16, XIN, DTP>(c) : launch_typed<1, 8, XIN, DTP>(c);
}

hipError_t launch_step(const StepCall& c) {
  if (c.dt_low) return launch_step_x<true, true>(c);  // dt_proj inside: an xc input only
  return c.xc_input ? launch_step_x<true, false>(c) : launch_step_x<false, false>(c);
}

}  // namespace mscan
