// One-token decode kernel of libmamba_scan for gfx950 (niverel-mamba 0.1.0
// PKG-INFO, "Autoregressive decoding": the step maps (states, token) to
// (output, new states); calm-mamba 0.1.4 PKG-INFO, O(1) state-cached
// generation). The arithmetic is the prefill's with one timestep: the conv
// window is (conv_state[0..2], x), the new conv state drops the oldest entry.
//
// One lane per (b, d) channel. Each lane reads its own conv and SSM state and
// writes its own new ones, after all reads, so in-place updates are safe.
// The step moves ~160 bytes of state per channel and does O(d_state) math,
// so it is bound by HBM bandwidth.
#include "scan_device.h"
#include "scan_internal.h"

namespace mscan {

namespace {

constexpr int kBlock = 256;

template <int IO, int N>
__global__ __launch_bounds__(kBlock) void scan_step_kernel(
    int32_t batch, int32_t d_inner, const typename Io<IO>::T* __restrict__ x,
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

  const float c0 = conv_state_in[i * 3 + 0];
  const float c1 = conv_state_in[i * 3 + 1];
  const float c2 = conv_state_in[i * 3 + 2];
  float h[N];
#pragma unroll
  for (int n = 0; n < N; ++n) h[n] = ssm_state_in[i * N + n];

  const float xv = Io<IO>::load(x + i);
  float u = fmaf(conv_w[d * 4 + 0], c0, conv_b[d]);
  u = fmaf(conv_w[d * 4 + 1], c1, u);
  u = fmaf(conv_w[d * 4 + 2], c2, u);
  u = fmaf(conv_w[d * 4 + 3], xv, u);
  const float xc = silu(u);
  const float delta = softplus(Io<IO>::load(dt + i) + dt_bias[d]);
  const float dx = delta * xc;
  const typename Io<IO>::T* Bt = Bm + static_cast<int64_t>(b) * N;
  const typename Io<IO>::T* Ct = Cm + static_cast<int64_t>(b) * N;
  float acc = 0.0f;
#pragma unroll
  for (int n = 0; n < N; ++n) {
    const float dA = exp2_hw(delta * (A[d * N + n] * kLog2e));
    h[n] = fmaf(dA, h[n], dx * Io<IO>::load(Bt + n));
    acc = fmaf(Io<IO>::load(Ct + n), h[n], acc);
  }
  const float out = fmaf(Dskip[d], xc, acc) * silu(Io<IO>::load(z + i));
  Io<IO>::store(y + i, out);

#pragma unroll
  for (int n = 0; n < N; ++n) ssm_state_out[i * N + n] = h[n];
  conv_state_out[i * 3 + 0] = c1;
  conv_state_out[i * 3 + 1] = c2;
  conv_state_out[i * 3 + 2] = xv;
}

template <int IO, int N>
hipError_t launch_typed(const StepCall& c) {
  using T = typename Io<IO>::T;
  const int64_t total = static_cast<int64_t>(c.batch) * c.d_inner;
  const dim3 grid(static_cast<unsigned>((total + kBlock - 1) / kBlock));
  hipLaunchKernelGGL((scan_step_kernel<IO, N>), grid, dim3(kBlock), 0, c.stream, c.batch, c.d_inner,
                     static_cast<const T*>(c.x), static_cast<const T*>(c.dt), static_cast<const T*>(c.z),
                     static_cast<const T*>(c.B), static_cast<const T*>(c.C), c.conv_w, c.conv_b, c.dt_bias,
                     c.D, c.A, c.conv_state_in, c.ssm_state_in, static_cast<T*>(c.y), c.conv_state_out,
                     c.ssm_state_out);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_step(const StepCall& c) {
  if (c.io_dtype == 0) return c.d_state == 16 ? launch_typed<0, 16>(c) : launch_typed<0, 8>(c);
  return c.d_state == 16 ? launch_typed<1, 16>(c) : launch_typed<1, 8>(c);
}

}  // namespace mscan
