// Issue-rate probe for gfx950: the measurement that sets the VALU roofline the
// prefill kernels are reported against. Not part of the scan library; it is
// built as libmamba_probe.so and driven by bench.py --valu-probe.
//
// Each kernel runs `iters` rounds of 32 float32 operations per lane on eight
// independent chains (or one dependent chain), with a chosen number of waves
// per SIMD (grid = 256 CUs x waves workgroups of 256 threads, i.e. one wave
// per SIMD per workgroup). The host times the launch with HIP events; the
// first workgroup also reads the shader clock counter (s_memtime) and the
// constant-rate wall clock (s_memrealtime) around its loop, so the clock the
// SIMDs ran at during the probe can be derived.
//
// Kinds: 0 = independent FMA, 1 = independent exp2 (v_exp_f32), 2 = one exp2
// per three FMA, 3 = a single dependent FMA chain, 4 = log2 (v_log_f32),
// 5 = reciprocal (v_rcp_f32), 6 = multiplies whose first operand is a DPP row
// broadcast (v_mul_f32 with row_newbcast), 7 = plain multiplies (the same
// data flow without DPP); with the encoding fixed by inline asm and every
// operand in a VGPR: 8 = v_add_f32_e32, 9 = v_fmac_f32_e32, 10 = v_fma_f32
// (VOP3), 11 = v_mul_f32_e64 (VOP3), 12 = v_mul_f32_e32; 13 = one exp2 per
// three plain multiplies.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

template <int J>
__device__ __forceinline__ float bcast(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x150 + J, 0xF, 0xF, true));
}
__device__ __forceinline__ float bcast_j(float v, int j) {
  switch (j & 7) {
    case 0: return bcast<0>(v);
    case 1: return bcast<1>(v);
    case 2: return bcast<2>(v);
    case 3: return bcast<3>(v);
    case 4: return bcast<4>(v);
    case 5: return bcast<5>(v);
    case 6: return bcast<6>(v);
    default: return bcast<7>(v);
  }
}

template <int KIND>
__global__ __launch_bounds__(256) void probe_kernel(int32_t iters, float m, float k, float* out, long long* clk) {
  const int tid = threadIdx.x;
  float a[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) a[c] = 0.25f + 1e-4f * static_cast<float>(tid + 37 * c);
  const float mv = m * (1.0f + 1e-9f * static_cast<float>(tid));  // a per-lane (VGPR) factor
  const float kv = k * (1.0f + 1e-9f * static_cast<float>(tid));  // a per-lane (VGPR) addend
  const long long t0 = clock64();
  const long long w0 = wall_clock64();
  for (int32_t i = 0; i < iters; ++i) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if (KIND == 0) {
#pragma unroll
        for (int c = 0; c < 8; ++c) a[c] = fmaf(a[c], m, k);
      } else if (KIND == 1) {
#pragma unroll
        for (int c = 0; c < 8; ++c) a[c] = __builtin_amdgcn_exp2f(-a[c]);
      } else if (KIND == 2) {
#pragma unroll
        for (int c = 0; c < 8; ++c) a[c] = (c % 4 == 0) ? __builtin_amdgcn_exp2f(-a[c]) : fmaf(a[c], m, k);
      } else if (KIND == 3) {
#pragma unroll
        for (int c = 0; c < 8; ++c) a[0] = fmaf(a[0], m, k);
      } else if (KIND == 6 || KIND == 7) {
        // a[c] = bcast(a[(c + 1) % 8], lane u*4 + c % 4) * m: every operand was
        // written at least seven instructions earlier
        float b[8];
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          const float src = a[(c + 1) % 8];
          const float v = KIND == 6 ? bcast_j(src, u * 4 + c) : src;
          b[c] = v * mv;
        }
#pragma unroll
        for (int c = 0; c < 8; ++c) a[c] = b[c];
      } else if (KIND >= 8 && KIND <= 12) {
        // one encoding pinned with inline asm (plain VALU arithmetic, no
        // memory access), eight independent accumulators
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          if (KIND == 8) asm volatile("v_add_f32_e32 %0, %1, %0" : "+v"(a[c]) : "v"(kv));
          if (KIND == 9) asm volatile("v_fmac_f32_e32 %0, %1, %2" : "+v"(a[c]) : "v"(mv), "v"(kv));
          if (KIND == 10) asm volatile("v_fma_f32 %0, %0, %1, %2" : "+v"(a[c]) : "v"(mv), "v"(kv));
          if (KIND == 11) asm volatile("v_mul_f32_e64 %0, %1, %0" : "+v"(a[c]) : "v"(mv));
          if (KIND == 12) asm volatile("v_mul_f32_e32 %0, %1, %0" : "+v"(a[c]) : "v"(mv));
        }
      } else if (KIND == 13) {
        // one exp2 per three plain multiplies
#pragma unroll
        for (int c = 0; c < 8; ++c) a[c] = (c % 4 == 0) ? __builtin_amdgcn_exp2f(-a[c]) : a[c] * mv;
      } else if (KIND == 4) {
#pragma unroll
        for (int c = 0; c < 8; ++c) a[c] = __builtin_amdgcn_logf(a[c] + 1.5f);
      } else if (KIND == 5) {
#pragma unroll
        for (int c = 0; c < 8; ++c) a[c] = __builtin_amdgcn_rcpf(a[c] + 1.5f);
      }
    }
  }
  const long long t1 = clock64();
  const long long w1 = wall_clock64();
  if (tid == 0 && blockIdx.x == 0) {
    clk[0] = t1 - t0;
    clk[1] = w1 - w0;
  }
  float s = 0.0f;
#pragma unroll
  for (int c = 0; c < 8; ++c) s += a[c];
  out[static_cast<size_t>(blockIdx.x) * 256 + tid] = s;
}

}  // namespace

extern "C" {

// Runs probe `kind` with `waves_per_simd` waves per SIMD (1..8) for `iters`
// rounds; writes the launch time (ms), the operations per lane it counts,
// and the shader-clock / wall-clock tick counts of the first workgroup.
// Returns 0, or a HIP error code. Allocates and frees its own buffers.
int mamba_probe_valu(int32_t kind, int32_t waves_per_simd, int32_t iters, float* ms_out,
                     double* ops_per_lane_out, long long* shader_ticks_out, long long* wall_ticks_out,
                     int32_t* wall_rate_khz_out) {
  if (kind < 0 || kind > 13 || waves_per_simd < 1 || waves_per_simd > 8 || iters < 1) return -1;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  int cus = 0, wall = 0;
  e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  e = hipDeviceGetAttribute(&wall, hipDeviceAttributeWallClockRate, dev);
  if (e != hipSuccess) return e;
  const unsigned blocks = static_cast<unsigned>(cus) * static_cast<unsigned>(waves_per_simd);
  float* out = nullptr;
  long long* clk = nullptr;
  if ((e = hipMalloc(&out, static_cast<size_t>(blocks) * 256 * sizeof(float))) != hipSuccess) return e;
  if ((e = hipMalloc(&clk, 2 * sizeof(long long))) != hipSuccess) {
    (void)hipFree(out);
    return e;
  }
  hipEvent_t e0, e1;
  (void)hipEventCreate(&e0);
  (void)hipEventCreate(&e1);
  auto launch = [&](int32_t it) {
    switch (kind) {
      case 0: hipLaunchKernelGGL(probe_kernel<0>, dim3(blocks), dim3(256), 0, 0, it, 0.999f, 1e-3f, out, clk); break;
      case 1: hipLaunchKernelGGL(probe_kernel<1>, dim3(blocks), dim3(256), 0, 0, it, 0.999f, 1e-3f, out, clk); break;
      case 2: hipLaunchKernelGGL(probe_kernel<2>, dim3(blocks), dim3(256), 0, 0, it, 0.999f, 1e-3f, out, clk); break;
      case 3: hipLaunchKernelGGL(probe_kernel<3>, dim3(blocks), dim3(256), 0, 0, it, 0.999f, 1e-3f, out, clk); break;
      case 4: hipLaunchKernelGGL(probe_kernel<4>, dim3(blocks), dim3(256), 0, 0, it, 0.999f, 1e-3f, out, clk); break;
      case 5: hipLaunchKernelGGL(probe_kernel<5>, dim3(blocks), dim3(256), 0, 0, it, 0.999f, 1e-3f, out, clk); break;
      case 6: hipLaunchKernelGGL(probe_kernel<6>, dim3(blocks), dim3(256), 0, 0, it, 0.999f, 1e-3f, out, clk); break;
      case 7: hipLaunchKernelGGL(probe_kernel<7>, dim3(blocks), dim3(256), 0, 0, it, 0.999f, 1e-3f, out, clk); break;
      case 8: hipLaunchKernelGGL(probe_kernel<8>, dim3(blocks), dim3(256), 0, 0, it, 0.999f, 1e-3f, out, clk); break;
      case 9: hipLaunchKernelGGL(probe_kernel<9>, dim3(blocks), dim3(256), 0, 0, it, 0.999f, 1e-3f, out, clk); break;
      case 10: hipLaunchKernelGGL(probe_kernel<10>, dim3(blocks), dim3(256), 0, 0, it, 0.999f, 1e-3f, out, clk); break;
      case 11: hipLaunchKernelGGL(probe_kernel<11>, dim3(blocks), dim3(256), 0, 0, it, 0.999f, 1e-3f, out, clk); break;
      case 12: hipLaunchKernelGGL(probe_kernel<12>, dim3(blocks), dim3(256), 0, 0, it, 0.999f, 1e-3f, out, clk); break;
      default: hipLaunchKernelGGL(probe_kernel<13>, dim3(blocks), dim3(256), 0, 0, it, 0.999f, 1e-3f, out, clk); break;
    }
  };
  launch(iters);  // warm-up
  (void)hipEventRecord(e0, 0);
  launch(iters);
  (void)hipEventRecord(e1, 0);
  e = hipEventSynchronize(e1);
  float ms = 0.0f;
  if (e == hipSuccess) e = hipEventElapsedTime(&ms, e0, e1);
  long long h[2] = {0, 0};
  if (e == hipSuccess) e = hipMemcpy(h, clk, sizeof h, hipMemcpyDeviceToHost);
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  (void)hipFree(out);
  (void)hipFree(clk);
  if (e != hipSuccess) return e;
  *ms_out = ms;
  *ops_per_lane_out = static_cast<double>(iters) * 32.0;
  *shader_ticks_out = h[0];
  *wall_ticks_out = h[1];
  *wall_rate_khz_out = wall;
  return 0;
}

}  // extern "C"
