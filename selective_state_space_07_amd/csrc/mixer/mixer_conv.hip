// Conv + SiLU feeding x_proj in the mixer layer of libmamba_mixer (calm-mamba
// 0.1.4 PKG-INFO, "Mamba operator", step 2): xc = SiLU(conv_b + sum_k
// conv_w[d][k] * xw[t-3+k]) with xw = conv history ++ x. The selective-scan
// kernels compute the same xc again internally; this copy (rounded to the io
// dtype) is only the input of the x_proj GEMM. One thread per output element;
// the four taps of a thread are consecutive rows of the same channel, so a
// wave's loads are coalesced across channels. HBM-bound.
#include "../scan_device.h"
#include "mixer_internal.h"

namespace mmix {

namespace {

using mscan::Io;
using mscan::silu;

constexpr int kBlock = 256;

template <int IO>
__global__ __launch_bounds__(kBlock) void conv_silu_kernel(int32_t seqlen, int32_t d_inner, int64_t total,
                                                           const typename Io<IO>::T* __restrict__ x,
                                                           const float* __restrict__ conv_w,
                                                           const float* __restrict__ conv_b,
                                                           const float* __restrict__ conv0,
                                                           typename Io<IO>::T* __restrict__ xc) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x;
  if (i >= total) return;
  const int32_t d = static_cast<int32_t>(i % d_inner);
  const int64_t bt = i / d_inner;
  const int32_t t = static_cast<int32_t>(bt % seqlen);
  const int64_t b = bt / seqlen;
  float u = conv_b[d];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int32_t tt = t - 3 + k;
    float v;
    if (tt >= 0) {
      v = Io<IO>::load(x + i + static_cast<int64_t>(tt - t) * d_inner);
    } else {
      v = conv0 ? conv0[(b * d_inner + d) * 3 + (3 + tt)] : 0.0f;
    }
    u = fmaf(conv_w[d * 4 + k], v, u);
  }
  Io<IO>::store(xc + i, silu(u));
}

// One token: the window is (conv_state[0..2], x).
template <int IO>
__global__ __launch_bounds__(kBlock) void conv_silu_step_kernel(int64_t total, int32_t d_inner,
                                                                const typename Io<IO>::T* __restrict__ x,
                                                                const float* __restrict__ conv_w,
                                                                const float* __restrict__ conv_b,
                                                                const float* __restrict__ cs,
                                                                typename Io<IO>::T* __restrict__ xc) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x;
  if (i >= total) return;
  const int32_t d = static_cast<int32_t>(i % d_inner);
  float u = conv_b[d];
  u = fmaf(conv_w[d * 4 + 0], cs[i * 3 + 0], u);
  u = fmaf(conv_w[d * 4 + 1], cs[i * 3 + 1], u);
  u = fmaf(conv_w[d * 4 + 2], cs[i * 3 + 2], u);
  u = fmaf(conv_w[d * 4 + 3], Io<IO>::load(x + i), u);
  Io<IO>::store(xc + i, silu(u));
}

}  // namespace

hipError_t launch_conv_silu(int io_dtype, int32_t batch, int32_t seqlen, int32_t d_inner, const void* x,
                            const float* conv_w, const float* conv_b, const float* conv0, void* xc,
                            hipStream_t stream) {
  const int64_t total = static_cast<int64_t>(batch) * seqlen * d_inner;
  const dim3 grid(static_cast<unsigned>((total + kBlock - 1) / kBlock));
  if (io_dtype == 0) {
    hipLaunchKernelGGL((conv_silu_kernel<0>), grid, dim3(kBlock), 0, stream, seqlen, d_inner, total,
                       static_cast<const float*>(x), conv_w, conv_b, conv0, static_cast<float*>(xc));
  } else {
    hipLaunchKernelGGL((conv_silu_kernel<1>), grid, dim3(kBlock), 0, stream, seqlen, d_inner, total,
                       static_cast<const uint16_t*>(x), conv_w, conv_b, conv0, static_cast<uint16_t*>(xc));
  }
  return hipGetLastError();
}

hipError_t launch_conv_silu_step(int io_dtype, int32_t batch, int32_t d_inner, const void* x, const float* conv_w,
                                 const float* conv_b, const float* conv_state, void* xc, hipStream_t stream) {
  const int64_t total = static_cast<int64_t>(batch) * d_inner;
  const dim3 grid(static_cast<unsigned>((total + kBlock - 1) / kBlock));
  if (io_dtype == 0) {
    hipLaunchKernelGGL((conv_silu_step_kernel<0>), grid, dim3(kBlock), 0, stream, total, d_inner,
                       static_cast<const float*>(x), conv_w, conv_b, conv_state, static_cast<float*>(xc));
  } else {
    hipLaunchKernelGGL((conv_silu_step_kernel<1>), grid, dim3(kBlock), 0, stream, total, d_inner,
                       static_cast<const uint16_t*>(x), conv_w, conv_b, conv_state, static_cast<uint16_t*>(xc));
  }
  return hipGetLastError();
}

}  // namespace mmix
