// Conv + SiLU in the mixer layer of libmamba_mixer (calm-mamba 0.1.4 PKG-INFO,
// "Mamba operator", step 2): xc = SiLU(conv_b + sum_k conv_w[d][k] *
// xw[t-3+k]) with xw = conv history ++ x, stored in the io dtype; it feeds
// both x_proj and, for a whole sequence, the scan (mamba_scan_fwd_xc), and
// the conv state after the last token is written here too. A thread takes one channel for
// kRows consecutive timesteps and slides the conv window down them in
// registers, so every x row is read once; consecutive threads take
// consecutive channels, so a wave's loads and stores are coalesced rows.
// Index arithmetic is done once per thread (no per-element 64-bit division).
// x is read from rows xs elements apart: d_inner, or in_proj's output rows
// (x, then z) of 2 * d_inner. HBM-bound.
#include "../scan_device.h"
#include "mixer_internal.h"

namespace mmix {

namespace {

using mscan::Io;
using mscan::silu;

constexpr int kBlock = 256;

constexpr int kRows = 16;  // timesteps per thread

// blockIdx.x: block of kBlock channels; blockIdx.y (grid-strided): one
// (batch row, block of kRows timesteps).
template <int IO>
__global__ __launch_bounds__(kBlock) void conv_silu_kernel(int32_t batch, int32_t seqlen, int32_t d_inner,
                                                           int32_t tblocks, const typename Io<IO>::T* __restrict__ x,
                                                           int32_t xs,
                                                           const float* __restrict__ conv_w,
                                                           const float* __restrict__ conv_b,
                                                           const float* __restrict__ conv0,
                                                           typename Io<IO>::T* __restrict__ xc) {
  const int32_t d = static_cast<int32_t>(blockIdx.x) * kBlock + static_cast<int32_t>(threadIdx.x);
  if (d >= d_inner) return;
  const float w0 = conv_w[d * 4], w1 = conv_w[d * 4 + 1], w2 = conv_w[d * 4 + 2], w3 = conv_w[d * 4 + 3];
  const float cb = conv_b[d];
  const int32_t ny = batch * tblocks;
  for (int32_t y = static_cast<int32_t>(blockIdx.y); y < ny; y += static_cast<int32_t>(gridDim.y)) {
    const int32_t b = y / tblocks, t0 = (y - b * tblocks) * kRows;
    const int64_t row0 = static_cast<int64_t>(b) * seqlen;
    // the window before t0: rows t0-3 .. t0-1, or the conv history before t = 0
    float v[3];
#pragma unroll
    for (int k = 0; k < 3; ++k) {
      const int32_t tt = t0 - 3 + k;
      if (tt >= 0) {
        v[k] = Io<IO>::load(x + (row0 + tt) * xs + d);
      } else {
        v[k] = conv0 ? conv0[(static_cast<int64_t>(b) * d_inner + d) * 3 + (3 + tt)] : 0.0f;
      }
    }
    // the block's rows, loaded first (rows past the end read the last row and
    // store nothing)
    const typename Io<IO>::T* xrow = x + row0 * xs + d;
    typename Io<IO>::T* ys = xc + row0 * d_inner + d;
    float xr[kRows];
#pragma unroll
    for (int j = 0; j < kRows; ++j) xr[j] = Io<IO>::load(xrow + static_cast<int64_t>(min(t0 + j, seqlen - 1)) * xs);
#pragma unroll
    for (int j = 0; j < kRows; ++j) {
      float u = cb;
      u = fmaf(w0, v[0], u);
      u = fmaf(w1, v[1], u);
      u = fmaf(w2, v[2], u);
      u = fmaf(w3, xr[j], u);
      if (t0 + j < seqlen) Io<IO>::store(ys + static_cast<int64_t>(t0 + j) * d_inner, silu(u));
      v[0] = v[1];
      v[1] = v[2];
      v[2] = xr[j];
    }
  }
}

// The conv state after the last token: entry j (0 = oldest) is element
// seqlen - 3 + j of (history ++ x), an exact copy (from the history when the
// sequence is shorter than 3). One thread per (batch row, channel); it reads
// its own history entries before writing, so the output may be the history
// array itself.
template <int IO>
__global__ __launch_bounds__(kBlock) void conv_state_kernel(int32_t batch, int32_t seqlen, int32_t d_inner,
                                                            const typename Io<IO>::T* __restrict__ x, int32_t xs,
                                                            const float* conv0, float* cso) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x;
  if (i >= static_cast<int64_t>(batch) * d_inner) return;
  const int64_t b = i / d_inner, d = i - b * d_inner;
  float v[3];
#pragma unroll
  for (int j = 0; j < 3; ++j) {
    const int32_t t = seqlen - 3 + j;
    v[j] = t >= 0 ? Io<IO>::load(x + (b * seqlen + t) * xs + d) : (conv0 ? conv0[i * 3 + 3 + t] : 0.0f);
  }
#pragma unroll
  for (int j = 0; j < 3; ++j) cso[i * 3 + j] = v[j];
}

// One token: the window is (conv_state[0..2], x); the new conv state
// (conv_state[1], conv_state[2], x) is written to cso, which may be the
// state array itself (each thread reads its entries before writing them).
// blockIdx.x: block of kBlock channels; blockIdx.y (grid-strided): batch row.
template <int IO>
__global__ __launch_bounds__(kBlock) void conv_silu_step_kernel(int32_t batch, int32_t d_inner,
                                                                const typename Io<IO>::T* __restrict__ x, int32_t xs,
                                                                const float* __restrict__ conv_w,
                                                                const float* __restrict__ conv_b, const float* cs,
                                                                typename Io<IO>::T* __restrict__ xc, float* cso) {
  const int32_t d = static_cast<int32_t>(blockIdx.x) * kBlock + static_cast<int32_t>(threadIdx.x);
  if (d >= d_inner) return;
  for (int32_t b = static_cast<int32_t>(blockIdx.y); b < batch; b += static_cast<int32_t>(gridDim.y)) {
    const int64_t i = static_cast<int64_t>(b) * d_inner + d;
    const float c0 = cs[i * 3 + 0], c1 = cs[i * 3 + 1], c2 = cs[i * 3 + 2];
    const float xv = Io<IO>::load(x + static_cast<int64_t>(b) * xs + d);
    float u = conv_b[d];
    u = fmaf(conv_w[d * 4 + 0], c0, u);
    u = fmaf(conv_w[d * 4 + 1], c1, u);
    u = fmaf(conv_w[d * 4 + 2], c2, u);
    u = fmaf(conv_w[d * 4 + 3], xv, u);
    Io<IO>::store(xc + i, silu(u));
    cso[i * 3 + 0] = c1;
    cso[i * 3 + 1] = c2;
    cso[i * 3 + 2] = xv;
  }
}

}  // namespace

hipError_t launch_conv_silu(int io_dtype, int32_t batch, int32_t seqlen, int32_t d_inner, const void* x, int32_t xs,
                            const float* conv_w, const float* conv_b, const float* conv0, void* xc,
                            hipStream_t stream) {
  if (batch < 1 || seqlen < 1 || d_inner < 1) return hipSuccess;
  const int32_t tblocks = (seqlen + kRows - 1) / kRows;
  const int64_t ny = static_cast<int64_t>(batch) * tblocks;
  const dim3 grid(static_cast<unsigned>((d_inner + kBlock - 1) / kBlock), static_cast<unsigned>(min(ny, int64_t{65535})));
  if (io_dtype == 0) {
    hipLaunchKernelGGL((conv_silu_kernel<0>), grid, dim3(kBlock), 0, stream, batch, seqlen, d_inner, tblocks,
                       static_cast<const float*>(x), xs, conv_w, conv_b, conv0, static_cast<float*>(xc));
  } else {
    hipLaunchKernelGGL((conv_silu_kernel<1>), grid, dim3(kBlock), 0, stream, batch, seqlen, d_inner, tblocks,
                       static_cast<const uint16_t*>(x), xs, conv_w, conv_b, conv0, static_cast<uint16_t*>(xc));
  }
  return hipGetLastError();
}

hipError_t launch_conv_state(int io_dtype, int32_t batch, int32_t seqlen, int32_t d_inner, const void* x, int32_t xs,
                             const float* conv0, float* cso, hipStream_t stream) {
  if (batch < 1 || seqlen < 1 || d_inner < 1 || cso == nullptr) return hipSuccess;
  const int64_t total = static_cast<int64_t>(batch) * d_inner;
  const dim3 grid(static_cast<unsigned>((total + kBlock - 1) / kBlock));
  if (io_dtype == 0) {
    hipLaunchKernelGGL((conv_state_kernel<0>), grid, dim3(kBlock), 0, stream, batch, seqlen, d_inner,
                       static_cast<const float*>(x), xs, conv0, cso);
  } else {
    hipLaunchKernelGGL((conv_state_kernel<1>), grid, dim3(kBlock), 0, stream, batch, seqlen, d_inner,
                       static_cast<const uint16_t*>(x), xs, conv0, cso);
  }
  return hipGetLastError();
}

hipError_t launch_conv_silu_step(int io_dtype, int32_t batch, int32_t d_inner, const void* x, int32_t xs,
                                 const float* conv_w, const float* conv_b, const float* conv_state, void* xc,
                                 float* conv_state_out, hipStream_t stream) {
  if (batch < 1 || d_inner < 1) return hipSuccess;
  const dim3 grid(static_cast<unsigned>((d_inner + kBlock - 1) / kBlock), static_cast<unsigned>(min(batch, 65535)));
  if (io_dtype == 0) {
    hipLaunchKernelGGL((conv_silu_step_kernel<0>), grid, dim3(kBlock), 0, stream, batch, d_inner,
                       static_cast<const float*>(x), xs, conv_w, conv_b, conv_state, static_cast<float*>(xc),
                       conv_state_out);
  } else {
    hipLaunchKernelGGL((conv_silu_step_kernel<1>), grid, dim3(kBlock), 0, stream, batch, d_inner,
                       static_cast<const uint16_t*>(x), xs, conv_w, conv_b, conv_state, static_cast<uint16_t*>(xc),
                       conv_state_out);
  }
  return hipGetLastError();
}

}  // namespace mmix
