// Backward of the prefill for gfx950 (d_state = 16): gradients of
// L = sum(y * dy) with respect to x, dt, z, B, C and the parameters, for the
// operation of calm-mamba 0.1.4 PKG-INFO, "Mamba operator", steps 2, 4, 5, 6
// (the page's kernels recompute the forward in their backward; so does this).
//
// Work layout: sixteen lanes per channel as in the prefill (lane n keeps state
// n; a 256-thread workgroup serves 16 channels of one batch row).
//  1. ckpt kernel: the forward recurrence, saving h before every stage of 16
//     timesteps ([batch][d_inner][stages][16] float32).
//  2. bwd kernel: the stages in reverse order. Per stage, the forward is
//     recomputed from the checkpoint (h of the 16 steps stays in VGPRs), then
//     the adjoint dh runs backwards through the 16 steps. Sums over the 16
//     states (the readout y, and the state's share of dxc and ddelta) are
//     row all-reductions by DPP rotations; each timestep's lane keeps its own.
//     The lane of timestep t then back-propagates through the gate, the
//     softplus, the SiLU and the conv; dx[t] needs du of t .. t+3, taken from
//     the next lanes and, across the stage edge, from the three first du of
//     the later stage (carried).
//     dB and dC (shared by all channels of a batch row) are summed over the
//     workgroup's channels through LDS and written as per-workgroup partials;
//     the parameter gradients are summed over the row's timesteps and written
//     per (batch row, channel).
//  3. reduce kernels: partials summed over workgroups (dB, dC) and over batch
//     rows (parameters), in a fixed order, so results are deterministic.
// Gradients with respect to the initial states are not produced.
#include "scan_device.h"
#include "scan_internal.h"

namespace mscan {

namespace {

constexpr int kThreads = 256;
constexpr int kN = 16;
constexpr int kCPB = kThreads / kN;  // channels per workgroup
constexpr int kStage = 16;
constexpr int kPG = 3 * kN;          // per-(b, d) parameter partials: dA[16], dconv_w[4], dconv_b, ddt_bias, dD, pad

__device__ __forceinline__ float sigmoid_hw(float v) { return rcp_hw(1.0f + exp2_hw(-v * kLog2e)); }

template <int J>
__device__ __forceinline__ float bcast(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x150 + J, 0xF, 0xF, true));
}
__device__ __forceinline__ float bcast_j(float v, int j) {
  switch (j) {
    case 0: return bcast<0>(v);
    case 1: return bcast<1>(v);
    case 2: return bcast<2>(v);
    case 3: return bcast<3>(v);
    case 4: return bcast<4>(v);
    case 5: return bcast<5>(v);
    case 6: return bcast<6>(v);
    case 7: return bcast<7>(v);
    case 8: return bcast<8>(v);
    case 9: return bcast<9>(v);
    case 10: return bcast<10>(v);
    case 11: return bcast<11>(v);
    case 12: return bcast<12>(v);
    case 13: return bcast<13>(v);
    case 14: return bcast<14>(v);
    default: return bcast<15>(v);
  }
}
// Sum over the 16 lanes of each row, in every lane of the row (rotations by
// 8, 4, 2, 1 within the row).
__device__ __forceinline__ float row_sum(float v) {
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x128, 0xF, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x124, 0xF, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x122, 0xF, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x121, 0xF, 0xF, false));
  return v;
}

// Workgroup blockIdx.x serves channel group g = blockIdx.x % groups of batch
// row b = blockIdx.x / groups (one grid dimension, so any batch fits).
struct Chan {
  int32_t b, g, d;
  bool active;
};
__device__ __forceinline__ Chan channel(int32_t d_inner, int32_t groups, int tid) {
  const int32_t blk = static_cast<int32_t>(blockIdx.x);
  const int32_t b = blk / groups, g = blk - b * groups;
  const int32_t d_raw = g * kCPB + (tid >> 4);
  return Chan{b, g, d_raw < d_inner ? d_raw : d_inner - 1, d_raw < d_inner};
}

// Per-element forward terms of timestep t of channel d.
struct Elem {
  float xw[4];  // conv window x[t-3 .. t] (history before 0)
  float u, xc, v, delta, dx;
};
template <int IO>
__device__ __forceinline__ Elem elem_at(int32_t t, int32_t seqlen, int32_t D, int32_t b, int32_t d,
                                        const typename Io<IO>::T* x, const typename Io<IO>::T* dt,
                                        const float* conv0, const float (&w)[4], float cb, float dtb) {
  Elem e;
  const size_t row0 = static_cast<size_t>(b) * seqlen;
  if (t < seqlen) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int32_t p = t - 3 + k;
      e.xw[k] = p >= 0 ? Io<IO>::load(x + (row0 + p) * D + d)
                       : (conv0 ? conv0[(static_cast<size_t>(b) * D + d) * 3 + 3 + p] : 0.0f);
    }
    e.v = Io<IO>::load(dt + (row0 + t) * D + d) + dtb;
  } else {
#pragma unroll
    for (int k = 0; k < 4; ++k) e.xw[k] = 0.0f;
    e.v = 0.0f;
  }
  float u = cb;
#pragma unroll
  for (int k = 0; k < 4; ++k) u = fmaf(w[k], e.xw[k], u);
  e.u = u;
  e.xc = silu(u);
  e.delta = softplus(e.v);
  e.dx = e.delta * e.xc;
  return e;
}

// 1. Forward with checkpoints: ckpt[b][d][s][n] = h before timestep 16 s.
template <int IO>
__global__ __launch_bounds__(kThreads) void bwd_ckpt_kernel(
    int32_t seqlen, int32_t d_inner, int32_t stages, int32_t groups, const typename Io<IO>::T* __restrict__ x,
    const typename Io<IO>::T* __restrict__ dt, const typename Io<IO>::T* __restrict__ Bm,
    const float* __restrict__ conv_w, const float* __restrict__ conv_b, const float* __restrict__ dt_bias,
    const float* __restrict__ A, const float* conv0, const float* h0, float* __restrict__ ckpt) {
  const int tid = threadIdx.x, n = tid & (kN - 1);
  const int32_t D = d_inner;
  const Chan c = channel(D, groups, tid);
  const int32_t d = c.d, b = c.b;
  const float w[4] = {conv_w[d * 4], conv_w[d * 4 + 1], conv_w[d * 4 + 2], conv_w[d * 4 + 3]};
  const float cb = conv_b[d], dtb = dt_bias[d], A2 = A[d * kN + n] * kLog2e;
  const size_t row0 = static_cast<size_t>(b) * seqlen;
  const size_t cbase = (static_cast<size_t>(b) * D + d) * stages;
  float h = h0 ? h0[(static_cast<size_t>(b) * D + d) * kN + n] : 0.0f;
  for (int32_t s = 0; s < stages; ++s) {
    const int32_t ts = s * kStage;
    if (c.active) ckpt[(cbase + s) * kN + n] = h;
    const Elem e = elem_at<IO>(ts + n, seqlen, D, b, d, x, dt, conv0, w, cb, dtb);
    for (int j = 0; j < kStage && ts + j < seqlen; ++j) {  // wave-uniform bound
      const float dj = bcast_j(e.delta, j), dxj = bcast_j(e.dx, j);
      const float Bj = Io<IO>::load(Bm + (row0 + ts + j) * kN + n);
      h = fmaf(exp2_hw(dj * A2), h, dxj * Bj);
    }
  }
}

// 2. Backward over the stages in reverse.
template <int IO>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void bwd_kernel(
    int32_t seqlen, int32_t d_inner, int32_t stages, int32_t groups, const typename Io<IO>::T* __restrict__ x,
    const typename Io<IO>::T* __restrict__ dt, const typename Io<IO>::T* __restrict__ z,
    const typename Io<IO>::T* __restrict__ Bm, const typename Io<IO>::T* __restrict__ Cm,
    const float* __restrict__ conv_w, const float* __restrict__ conv_b, const float* __restrict__ dt_bias,
    const float* __restrict__ Dskip, const float* __restrict__ A, const float* conv0,
    const float* __restrict__ ckpt, const typename Io<IO>::T* __restrict__ dy, typename Io<IO>::T* __restrict__ dx,
    typename Io<IO>::T* __restrict__ ddt, typename Io<IO>::T* __restrict__ dz,
    float* __restrict__ dBpart,  // [batch][groups][seqlen][16]
    float* __restrict__ dCpart,
    float* __restrict__ pgrad)   // [batch][d_inner][kPG]
{
  __shared__ float bc[2][kStage][kN + 4];               // B / C rows of the stage, [timestep][n]
  __shared__ float part[2][kCPB][kStage][kN + 1];       // dB / dC contributions, [channel][timestep][n]
  const int tid = threadIdx.x, n = tid & (kN - 1), cl = tid >> 4;
  const int32_t D = d_inner;
  const Chan c = channel(D, groups, tid);
  const int32_t d = c.d, b = c.b;
  const float w[4] = {conv_w[d * 4], conv_w[d * 4 + 1], conv_w[d * 4 + 2], conv_w[d * 4 + 3]};
  const float cb = conv_b[d], dtb = dt_bias[d], Dd = Dskip[d];
  const float An = A[d * kN + n], A2 = An * kLog2e;
  const size_t row0 = static_cast<size_t>(b) * seqlen;
  const size_t cbase = (static_cast<size_t>(b) * D + d) * stages;

  float dh = 0.0f;
  float g_dA = 0.0f, g_dD = 0.0f, g_dtb = 0.0f, g_cb = 0.0f, g_cw[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  float carry0 = 0.0f, carry1 = 0.0f, carry2 = 0.0f;  // du of the first three steps of the later stage

  for (int32_t s = stages - 1; s >= 0; --s) {
    const int32_t ts = s * kStage;
    const int nv = min(kStage, seqlen - ts);  // valid steps of this stage (wave-uniform)
    // B / C rows of the stage into LDS (element tid: timestep tid / 16, state tid % 16)
    __syncthreads();
    {
      const int tj = tid / kN, tn = tid % kN;
      const bool ok = tj < nv;
      bc[0][tj][tn] = ok ? Io<IO>::load(Bm + (row0 + ts + tj) * kN + tn) : 0.0f;
      bc[1][tj][tn] = ok ? Io<IO>::load(Cm + (row0 + ts + tj) * kN + tn) : 0.0f;
    }
    __syncthreads();
    // own timestep t = ts + n
    const int32_t t = ts + n;
    const bool valid = n < nv;
    const Elem e = elem_at<IO>(t, seqlen, D, b, d, x, dt, conv0, w, cb, dtb);
    float zt = 0.0f, dyt = 0.0f;
    if (valid) {
      zt = Io<IO>::load(z + (row0 + t) * D + d);
      dyt = Io<IO>::load(dy + (row0 + t) * D + d);
    }
    const float sz = sigmoid_hw(zt);
    const float gz = zt * sz;
    const float dyr = dyt * gz;  // dL/d(pre-gate y)
    float Bv[kStage], Cv[kStage];
#pragma unroll
    for (int j = 0; j < kStage; ++j) {
      Bv[j] = bc[0][j][n];
      Cv[j] = bc[1][j][n];
    }
    // forward recompute of the stage from its checkpoint
    const float hprev = ckpt[(cbase + s) * kN + n];
    float H[kStage], a[kStage];
    float yr_me = 0.0f;
    float h = hprev;
#pragma unroll
    for (int j = 0; j < kStage; ++j) {
      const float dj = bcast_j(e.delta, j), dxj = bcast_j(e.dx, j);
      a[j] = exp2_hw(dj * A2);
      h = (j < nv) ? fmaf(a[j], h, dxj * Bv[j]) : h;
      H[j] = h;
      const float yj = row_sum(Cv[j] * h);  // readout of step j (its C.h part)
      yr_me = (n == j) ? yj : yr_me;
    }
    const float yraw = fmaf(Dd, e.xc, yr_me);
    // adjoint through the 16 steps, newest first
    float T_me = 0.0f, S_me = 0.0f;
#pragma unroll
    for (int j = kStage - 1; j >= 0; --j) {
      if (j < nv) {  // wave-uniform
        const float dyrj = bcast_j(dyr, j), dxj = bcast_j(e.dx, j), dj = bcast_j(e.delta, j);
        dh = fmaf(Cv[j], dyrj, dh);
        part[1][cl][j][n] = H[j] * dyrj;                       // dC contribution
        const float hp = j > 0 ? H[j - 1] : hprev;
        const float ah = a[j] * hp;
        const float Tj = row_sum(dh * (An * ah));             // state's share of ddelta (decay term)
        const float Sj = row_sum(dh * Bv[j]);                  // sum_n dh B (input term, per unit delta*xc)
        T_me = (n == j) ? Tj : T_me;
        S_me = (n == j) ? Sj : S_me;
        part[0][cl][j][n] = dh * dxj;                          // dB contribution
        g_dA = fmaf(dh * dj, ah, g_dA);
        dh *= a[j];
      } else {
        part[0][cl][j][n] = 0.0f;
        part[1][cl][j][n] = 0.0f;
      }
    }
    // element backward of the own timestep
    float du = 0.0f;
    if (valid) {
      if (c.active) {
        Io<IO>::store(dz + (row0 + t) * D + d, dyt * yraw * sz * (1.0f + zt * (1.0f - sz)));
      }
      g_dD = fmaf(dyr, e.xc, g_dD);
      const float dxc = fmaf(dyr, Dd, e.delta * S_me);
      const float ddelta = fmaf(e.xc, S_me, T_me);
      const float dv = ddelta * sigmoid_hw(e.v);
      if (c.active) Io<IO>::store(ddt + (row0 + t) * D + d, dv);
      g_dtb += dv;
      const float su = sigmoid_hw(e.u);
      du = dxc * su * (1.0f + e.u * (1.0f - su));
      g_cb += du;
#pragma unroll
      for (int k = 0; k < 4; ++k) g_cw[k] = fmaf(du, e.xw[k], g_cw[k]);
    }
    // dx[t] = w3 du[t] + w2 du[t+1] + w1 du[t+2] + w0 du[t+3]
    const float du1 = __shfl_down(du, 1, kN), du2 = __shfl_down(du, 2, kN), du3 = __shfl_down(du, 3, kN);
    const float n1 = n + 1 < kN ? du1 : carry0;
    const float n2 = n + 2 < kN ? du2 : (n == 14 ? carry0 : carry1);
    const float n3 = n + 3 < kN ? du3 : (n == 13 ? carry0 : (n == 14 ? carry1 : carry2));
    if (valid && c.active) {
      const float gx = fmaf(w[0], n3, fmaf(w[1], n2, fmaf(w[2], n1, w[3] * du)));
      Io<IO>::store(dx + (row0 + t) * D + d, gx);
    }
    carry0 = bcast<0>(du);
    carry1 = bcast<1>(du);
    carry2 = bcast<2>(du);
    // dB / dC of the stage summed over the workgroup's channels
    __syncthreads();
    {
      const int tj = tid / kN, tn = tid % kN;
      if (tj < nv) {
        float sb = 0.0f, sc = 0.0f;
        for (int k = 0; k < kCPB; ++k) {
          const bool chan_ok = c.g * kCPB + k < D;
          sb += chan_ok ? part[0][k][tj][tn] : 0.0f;
          sc += chan_ok ? part[1][k][tj][tn] : 0.0f;
        }
        const size_t o = ((static_cast<size_t>(b) * groups + c.g) * seqlen + ts + tj) * kN + tn;
        dBpart[o] = sb;
        dCpart[o] = sc;
      }
    }
  }
  // parameter partials of this (b, d): lane n holds dA[n]; the rest is summed over the row
  g_dD = row_sum(g_dD);
  g_dtb = row_sum(g_dtb);
  g_cb = row_sum(g_cb);
#pragma unroll
  for (int k = 0; k < 4; ++k) g_cw[k] = row_sum(g_cw[k]);
  if (c.active) {
    float* pg = pgrad + (static_cast<size_t>(b) * D + d) * kPG;
    pg[n] = g_dA;
    if (n < 4) pg[kN + n] = g_cw[n];
    if (n == 4) pg[kN + 4] = g_cb;
    if (n == 5) pg[kN + 5] = g_dtb;
    if (n == 6) pg[kN + 6] = g_dD;
  }
}

// 3a. dB[b][t][n] = sum over workgroups of the partials, in workgroup order.
__global__ __launch_bounds__(kThreads) void bwd_reduce_bc_kernel(int64_t total, int32_t seqlen, int32_t groups,
                                                                 const float* __restrict__ pB,
                                                                 const float* __restrict__ pC, float* __restrict__ dB,
                                                                 float* __restrict__ dC) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;  // (b, t, n)
  if (i >= total) return;
  const int64_t per_b = static_cast<int64_t>(seqlen) * kN;
  const int64_t b = i / per_b, r = i - b * per_b;
  float sb = 0.0f, sc = 0.0f;
  for (int32_t g = 0; g < groups; ++g) {
    const int64_t o = (b * groups + g) * per_b + r;
    sb += pB[o];
    sc += pC[o];
  }
  dB[i] = sb;
  dC[i] = sc;
}

// 3b. parameter gradients summed over batch rows, in row order.
__global__ __launch_bounds__(kThreads) void bwd_reduce_params_kernel(int32_t batch, int32_t d_inner,
                                                                     const float* __restrict__ pg, float* dconv_w,
                                                                     float* dconv_b, float* ddt_bias, float* dD,
                                                                     float* dA) {
  const int32_t i = blockIdx.x * kThreads + threadIdx.x;  // (d, field)
  if (i >= d_inner * (kN + 7)) return;
  const int32_t d = i / (kN + 7), f = i % (kN + 7);
  float s = 0.0f;
  for (int32_t b = 0; b < batch; ++b) s += pg[(static_cast<size_t>(b) * d_inner + d) * kPG + f];
  if (f < kN) {
    dA[d * kN + f] = s;
  } else if (f < kN + 4) {
    dconv_w[d * 4 + (f - kN)] = s;
  } else if (f == kN + 4) {
    dconv_b[d] = s;
  } else if (f == kN + 5) {
    ddt_bias[d] = s;
  } else {
    dD[d] = s;
  }
}

template <int IO>
hipError_t launch_typed(const BwdCall& c) {
  using T = typename Io<IO>::T;
  const BwdWs w = bwd_ws_layout(c.batch, c.seqlen, c.d_inner);
  const int32_t stages = (c.seqlen + kStage - 1) / kStage;
  const int32_t groups = (c.d_inner + kCPB - 1) / kCPB;
  float* ckpt = c.workspace + w.ckpt;
  float* pB = c.workspace + w.dBpart;
  float* pC = c.workspace + w.dCpart;
  float* pg = c.workspace + w.pgrad;
  const dim3 grid(static_cast<unsigned>(groups) * static_cast<unsigned>(c.batch));
  hipLaunchKernelGGL((bwd_ckpt_kernel<IO>), grid, dim3(kThreads), 0, c.stream, c.seqlen, c.d_inner, stages, groups,
                     static_cast<const T*>(c.x), static_cast<const T*>(c.dt), static_cast<const T*>(c.B), c.conv_w,
                     c.conv_b, c.dt_bias, c.A, c.conv_state_in, c.ssm_state_in, ckpt);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((bwd_kernel<IO>), grid, dim3(kThreads), 0, c.stream, c.seqlen, c.d_inner, stages, groups,
                     static_cast<const T*>(c.x), static_cast<const T*>(c.dt), static_cast<const T*>(c.z),
                     static_cast<const T*>(c.B), static_cast<const T*>(c.C), c.conv_w, c.conv_b, c.dt_bias, c.D, c.A,
                     c.conv_state_in, ckpt, static_cast<const T*>(c.dy), static_cast<T*>(c.dx),
                     static_cast<T*>(c.ddt), static_cast<T*>(c.dz), pB, pC, pg);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t total = static_cast<int64_t>(c.batch) * c.seqlen * kN;
  hipLaunchKernelGGL(bwd_reduce_bc_kernel, dim3(static_cast<unsigned>((total + kThreads - 1) / kThreads)),
                     dim3(kThreads), 0, c.stream, total, c.seqlen, groups, pB, pC, c.dB, c.dC);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int32_t np = c.d_inner * (kN + 7);
  hipLaunchKernelGGL(bwd_reduce_params_kernel, dim3(static_cast<unsigned>((np + kThreads - 1) / kThreads)),
                     dim3(kThreads), 0, c.stream, c.batch, c.d_inner, pg, c.dconv_w, c.dconv_b, c.ddt_bias, c.dD,
                     c.dA);
  return hipGetLastError();
}

}  // namespace

BwdWs bwd_ws_layout(int32_t batch, int32_t seqlen, int32_t d_inner) {
  BwdWs w{};
  const size_t stages = (static_cast<size_t>(seqlen) + kStage - 1) / kStage;
  const size_t groups = (static_cast<size_t>(d_inner) + kCPB - 1) / kCPB;
  w.ckpt = 0;
  w.dBpart = w.ckpt + static_cast<size_t>(batch) * d_inner * stages * kN;
  w.dCpart = w.dBpart + static_cast<size_t>(batch) * groups * seqlen * kN;
  w.pgrad = w.dCpart + static_cast<size_t>(batch) * groups * seqlen * kN;
  w.total = w.pgrad + static_cast<size_t>(batch) * d_inner * kPG;
  return w;
}

hipError_t launch_bwd(const BwdCall& c) {
  return c.io_dtype == 0 ? launch_typed<0>(c) : launch_typed<1>(c);
}

}  // namespace mscan
