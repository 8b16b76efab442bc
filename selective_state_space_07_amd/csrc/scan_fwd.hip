// Prefill kernels of libmamba_scan for gfx950.
//
// Computes, for every batch row b and channel d (calm-mamba 0.1.4 PKG-INFO,
// "Mamba operator", steps 2, 4, 5, 6): the causal depthwise conv (4 taps) +
// SiLU, delta = softplus(dt + dt_bias), the recurrence
// h = exp(delta*A)*h + delta*B*xc with readout C.h + D*xc, and the SiLU(z)
// gate; plus the final conv and SSM states.
//
// Layout of the work: one lane per (b, d) channel, the d_state values of h in
// VGPRs, 64 consecutive channels of one batch row per wave, so that the
// B[t] and C[t] rows (shared by every channel) are wave-uniform and come in
// through scalar loads into SGPRs, and the x/dt/z/y accesses of a wave are
// contiguous along d.
//
// The sequence is split into chunks when the channels alone cannot fill the
// 1024 SIMDs. The recurrence is affine in h, so a chunk's effect on the state
// is the pair (P, S): P[n] = exp(A[n] * sum of its deltas) and S = its end
// state when started from zero. Pairs compose associatively (not
// commutatively): the state after chunks 0..c is P_c*(...(P_0*h_init + S_0)...)
// + S_c. Pass 1 (kSummary) computes (sum delta, S) for every chunk but the
// last; pass 2 (kFinal) folds the summaries of the chunks before its own into
// its carry-in, then runs its chunk producing y (and, in the last chunk, the
// final states). Pass 1 also copies the incoming states into the workspace,
// so pass 2 never reads a state buffer that the last chunk may overwrite in
// place.
#include <cstdlib>
#include <cstring>

#include "scan_device.h"
#include "scan_internal.h"

namespace mscan {

namespace {

constexpr int kWave = 64;
constexpr int kConvHist = 3;  // d_conv - 1
constexpr int kMinChunk = 64;
#ifndef MSCAN_TARGET_WAVES
#define MSCAN_TARGET_WAVES 2048
#endif
#ifndef MSCAN_PREFETCH
#define MSCAN_PREFETCH 8
#endif
constexpr int kTargetWaves = MSCAN_TARGET_WAVES;  // waves a prefill launch aims for (1024 SIMDs)
constexpr int kPrefetch = MSCAN_PREFETCH;         // timesteps of x/dt/z loaded ahead of use

// Workspace layout (float32):
//   bc stage   [2][batch][seqlen][d_state]  B then C as float32 (bfloat16 io only)
//   summaries  [batch][n_chunks-1][d_state+1][d_inner]  (S[0..N-1], then sum delta)
//   ssm stash  [batch][d_state][d_inner]
//   conv stash [batch][3][d_inner]
// The last three exist only when the sequence is split; they are indexed with
// d fastest so that a wave's accesses are contiguous.
struct WsLayout {
  size_t bc_stage, summaries, ssm_stash, conv_stash, total;
};

__host__ __device__ inline WsLayout ws_layout(int32_t batch, int32_t seqlen, int32_t d_inner, int32_t d_state,
                                              int32_t n_chunks, bool stage_bc) {
  WsLayout w;
  const size_t bd = static_cast<size_t>(batch) * d_inner;
  const size_t bc = stage_bc ? 2 * static_cast<size_t>(batch) * seqlen * d_state : 0;
  w.bc_stage = 0;
  w.summaries = bc;
  if (n_chunks > 1) {
    w.ssm_stash = w.summaries + bd * static_cast<size_t>(n_chunks - 1) * (d_state + 1);
    w.conv_stash = w.ssm_stash + bd * d_state;
    w.total = w.conv_stash + bd * kConvHist;
  } else {
    w.ssm_stash = w.conv_stash = w.total = bc;
  }
  return w;
}

// B and C rows are read by every wave of a batch row; they are read through
// the constant address space so that the compiler emits scalar loads into
// SGPRs (they are never written while the kernels run).
typedef const __attribute__((address_space(4))) float* ConstRow;

// bfloat16 -> float32 copy of B and C into the staging area, 4 elements a
// thread; `count` = batch*seqlen*d_state (a multiple of 8).
__global__ __launch_bounds__(256) void stage_bc_kernel(const uint16_t* __restrict__ Bm,
                                                       const uint16_t* __restrict__ Cm, float* __restrict__ out,
                                                       int64_t count) {
  const int64_t i = (static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x) * 4;
  if (i >= 2 * count) return;
  const uint16_t* src = i < count ? Bm + i : Cm + (i - count);
#pragma unroll
  for (int k = 0; k < 4; ++k) out[i + k] = Io<1>::load(src + k);
}

enum Pass { kSummary = 0, kFinal = 1 };

template <int IO, int N, int PASS>
__global__ __launch_bounds__(kWave) void scan_fwd_kernel(
    int32_t seqlen, int32_t d_inner, int32_t n_chunks, int32_t chunk_len,
    const typename Io<IO>::T* __restrict__ x, const typename Io<IO>::T* __restrict__ dt,
    const typename Io<IO>::T* __restrict__ z, const float* __restrict__ Bm,
    const float* __restrict__ Cm, const float* __restrict__ conv_w,
    const float* __restrict__ conv_b, const float* __restrict__ dt_bias,
    const float* __restrict__ Dskip, const float* __restrict__ A,
    const float* __restrict__ conv_state_in, const float* __restrict__ ssm_state_in,
    typename Io<IO>::T* __restrict__ y, float* __restrict__ conv_state_out,
    float* __restrict__ ssm_state_out, float* __restrict__ ws) {
  using T = typename Io<IO>::T;
  const int32_t d_raw = blockIdx.x * kWave + threadIdx.x;
  const bool active = d_raw < d_inner;
  const int32_t d = active ? d_raw : d_inner - 1;  // inactive lanes mirror a valid channel, store nothing
  const int32_t chunk = blockIdx.y;
  const int32_t b = blockIdx.z;
  const int32_t t0 = chunk * chunk_len;
  const int32_t t1 = min(t0 + chunk_len, seqlen);
  const int32_t D = d_inner;
  const int32_t batch = gridDim.z;
  const WsLayout wl = ws_layout(batch, seqlen, d_inner, N, n_chunks, IO == 1);
  const size_t bd = static_cast<size_t>(b) * D + d;

  const float w0 = conv_w[d * 4 + 0], w1 = conv_w[d * 4 + 1], w2 = conv_w[d * 4 + 2], w3 = conv_w[d * 4 + 3];
  const float cb = conv_b[d];
  const float dtb = dt_bias[d];
  float A2[N];  // A * log2(e): exp(delta*A) = exp2(delta*A2)
#pragma unroll
  for (int n = 0; n < N; ++n) A2[n] = A[d * N + n] * kLog2e;

  // Conv history xh0 (oldest) .. xh2 (newest) before t0, and the carry-in h.
  float xh0, xh1, xh2;
  float h[N];
  const bool split = n_chunks > 1;
  if (chunk == 0) {
    float cs[kConvHist];
    float hs[N];
    if (PASS == kFinal && split) {  // pass 1 stashed the incoming states
#pragma unroll
      for (int j = 0; j < kConvHist; ++j) cs[j] = ws[wl.conv_stash + (static_cast<size_t>(b) * kConvHist + j) * D + d];
#pragma unroll
      for (int n = 0; n < N; ++n) hs[n] = ws[wl.ssm_stash + (static_cast<size_t>(b) * N + n) * D + d];
    } else {
#pragma unroll
      for (int j = 0; j < kConvHist; ++j) cs[j] = conv_state_in ? conv_state_in[bd * kConvHist + j] : 0.0f;
#pragma unroll
      for (int n = 0; n < N; ++n) hs[n] = ssm_state_in ? ssm_state_in[bd * N + n] : 0.0f;
      if (PASS == kSummary && active) {
#pragma unroll
        for (int j = 0; j < kConvHist; ++j) ws[wl.conv_stash + (static_cast<size_t>(b) * kConvHist + j) * D + d] = cs[j];
#pragma unroll
        for (int n = 0; n < N; ++n) ws[wl.ssm_stash + (static_cast<size_t>(b) * N + n) * D + d] = hs[n];
      }
    }
    xh0 = cs[0];
    xh1 = cs[1];
    xh2 = cs[2];
#pragma unroll
    for (int n = 0; n < N; ++n) h[n] = (PASS == kFinal) ? hs[n] : 0.0f;
  } else {
    // chunk_len >= kMinChunk > 3, so the history lies inside x.
    const size_t e = (static_cast<size_t>(b) * seqlen + t0) * D + d;
    xh0 = Io<IO>::load(x + e - 3 * static_cast<size_t>(D));
    xh1 = Io<IO>::load(x + e - 2 * static_cast<size_t>(D));
    xh2 = Io<IO>::load(x + e - 1 * static_cast<size_t>(D));
    if (PASS == kFinal) {
      // Carry-in: fold the stashed initial state through the summaries of
      // chunks 0 .. chunk-1, oldest first.
#pragma unroll
      for (int n = 0; n < N; ++n) h[n] = ws[wl.ssm_stash + (static_cast<size_t>(b) * N + n) * D + d];
      for (int32_t j = 0; j < chunk; ++j) {
        const float* s = ws + wl.summaries + (static_cast<size_t>(b) * (n_chunks - 1) + j) * (N + 1) * D + d;
        const float sum_delta = s[static_cast<size_t>(N) * D];
#pragma unroll
        for (int n = 0; n < N; ++n) h[n] = fmaf(exp2_hw(sum_delta * A2[n]), h[n], s[static_cast<size_t>(n) * D]);
      }
    } else {
#pragma unroll
      for (int n = 0; n < N; ++n) h[n] = 0.0f;
    }
  }

  const float dsk = (PASS == kFinal) ? Dskip[d] : 0.0f;
  float sum_delta = 0.0f;
  const size_t row = static_cast<size_t>(b) * seqlen;
  const uint32_t ld = static_cast<uint32_t>(d);
  const ConstRow Bs = (ConstRow)(Bm) + (row + t0) * N;
  const ConstRow Cs = (ConstRow)(Cm) + (row + t0) * N;
  // Wave-uniform row pointers of timestep t0; lanes add their channel d.
  const T* xr = x + (row + t0) * D;
  const T* dtr = dt + (row + t0) * D;
  const T* zr = z + (row + t0) * D;
  T* yr = y + (row + t0) * D;
  const int32_t len = t1 - t0;

  // x/dt/z of timesteps i .. i+P-1 (relative to t0) sit in a ring of P
  // registers per stream, refilled P steps ahead of use.
  T xq[kPrefetch], dq[kPrefetch], zq[kPrefetch];
#pragma unroll
  for (int j = 0; j < kPrefetch; ++j) {
    if (j < len) {
      const uint32_t o = static_cast<uint32_t>(j) * static_cast<uint32_t>(D) + ld;
      xq[j] = xr[o];
      dq[j] = dtr[o];
      if (PASS == kFinal) zq[j] = zr[o];
    }
  }
  // B and C rows of the next timestep, loaded one step ahead into SGPRs.
  float Bn[N], Cn[N];
#pragma unroll
  for (int n = 0; n < N; ++n) {
    Bn[n] = Bs[n];
    if (PASS == kFinal) Cn[n] = Cs[n];
  }

  // One timestep i (relative to t0) whose inputs are in ring slot j.
  auto step = [&](int32_t i, int j) {
    const float xv = Io<IO>::cvt(xq[j]);
    const float dv = Io<IO>::cvt(dq[j]);
    const float zv = (PASS == kFinal) ? Io<IO>::cvt(zq[j]) : 0.0f;
    const int32_t ir = i + kPrefetch;
    if (ir < len) {  // wave-uniform
      const uint32_t o = static_cast<uint32_t>(ir) * static_cast<uint32_t>(D) + ld;
      xq[j] = xr[o];
      dq[j] = dtr[o];
      if (PASS == kFinal) zq[j] = zr[o];
    }
    float Bv[N], Cv[N];
#pragma unroll
    for (int n = 0; n < N; ++n) {
      Bv[n] = Bn[n];
      if (PASS == kFinal) Cv[n] = Cn[n];
    }
    const size_t nxt = static_cast<size_t>(i + 1 < len ? i + 1 : i) * N;
#pragma unroll
    for (int n = 0; n < N; ++n) {
      Bn[n] = Bs[nxt + n];
      if (PASS == kFinal) Cn[n] = Cs[nxt + n];
    }
    // conv: tap 3 meets the newest input
    float u = fmaf(w0, xh0, cb);
    u = fmaf(w1, xh1, u);
    u = fmaf(w2, xh2, u);
    u = fmaf(w3, xv, u);
    xh0 = xh1;
    xh1 = xh2;
    xh2 = xv;
    const float xc = silu(u);
    const float delta = softplus(dv + dtb);
    const float dx = delta * xc;
    if (PASS == kFinal) {
      float acc = 0.0f;
#pragma unroll
      for (int n = 0; n < N; ++n) {
        const float dA = exp2_hw(delta * A2[n]);
        h[n] = fmaf(dA, h[n], dx * Bv[n]);
        acc = fmaf(Cv[n], h[n], acc);
      }
      const float out = fmaf(dsk, xc, acc) * silu(zv);
      if (active) Io<IO>::store(yr + static_cast<uint32_t>(i) * static_cast<uint32_t>(D) + ld, out);
    } else {
#pragma unroll
      for (int n = 0; n < N; ++n) {
        const float dA = exp2_hw(delta * A2[n]);
        h[n] = fmaf(dA, h[n], dx * Bv[n]);
      }
      sum_delta += delta;
    }
  };

  int32_t i = 0;
  for (; i + kPrefetch <= len; i += kPrefetch) {
#pragma unroll
    for (int j = 0; j < kPrefetch; ++j) step(i + j, j);
  }
#pragma unroll
  for (int j = 0; j < kPrefetch; ++j)
    if (i + j < len) step(i + j, j);

  if (!active) return;
  if (PASS == kSummary) {
    float* s = ws + wl.summaries + (static_cast<size_t>(b) * (n_chunks - 1) + chunk) * (N + 1) * D + d;
#pragma unroll
    for (int n = 0; n < N; ++n) s[static_cast<size_t>(n) * D] = h[n];
    s[static_cast<size_t>(N) * D] = sum_delta;
  } else if (chunk == n_chunks - 1) {
    if (ssm_state_out) {
#pragma unroll
      for (int n = 0; n < N; ++n) ssm_state_out[bd * N + n] = h[n];
    }
    if (conv_state_out) {
      conv_state_out[bd * kConvHist + 0] = xh0;
      conv_state_out[bd * kConvHist + 1] = xh1;
      conv_state_out[bd * kConvHist + 2] = xh2;
    }
  }
}

template <int IO, int N>
hipError_t launch_typed(const FwdCall& c, const FwdPlan& p) {
  using T = typename Io<IO>::T;
  const dim3 block(kWave);
  const unsigned dblocks = static_cast<unsigned>((c.d_inner + kWave - 1) / kWave);
  const T* x = static_cast<const T*>(c.x);
  const T* dt = static_cast<const T*>(c.dt);
  const T* z = static_cast<const T*>(c.z);
  const float* Bm = static_cast<const float*>(c.B);
  const float* Cm = static_cast<const float*>(c.C);
  T* y = static_cast<T*>(c.y);
  if (IO == 1) {  // stage B and C as float32
    const int64_t count = static_cast<int64_t>(c.batch) * c.seqlen * N;
    const WsLayout wl = ws_layout(c.batch, c.seqlen, c.d_inner, N, p.n_chunks, true);
    float* stage = c.workspace + wl.bc_stage;
    const int64_t threads = (2 * count + 3) / 4;
    hipLaunchKernelGGL(stage_bc_kernel, dim3(static_cast<unsigned>((threads + 255) / 256)), dim3(256), 0,
                       c.stream, static_cast<const uint16_t*>(c.B), static_cast<const uint16_t*>(c.C), stage, count);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    Bm = stage;
    Cm = stage + count;
  }
  if (p.n_chunks > 1) {
    const dim3 grid1(dblocks, static_cast<unsigned>(p.n_chunks - 1), static_cast<unsigned>(c.batch));
    hipLaunchKernelGGL((scan_fwd_kernel<IO, N, kSummary>), grid1, block, 0, c.stream, c.seqlen, c.d_inner,
                       p.n_chunks, p.chunk_len, x, dt, z, Bm, Cm, c.conv_w, c.conv_b, c.dt_bias, c.D, c.A,
                       c.conv_state_in, c.ssm_state_in, y, c.conv_state_out, c.ssm_state_out, c.workspace);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  const dim3 grid2(dblocks, static_cast<unsigned>(p.n_chunks), static_cast<unsigned>(c.batch));
  hipLaunchKernelGGL((scan_fwd_kernel<IO, N, kFinal>), grid2, block, 0, c.stream, c.seqlen, c.d_inner,
                     p.n_chunks, p.chunk_len, x, dt, z, Bm, Cm, c.conv_w, c.conv_b, c.dt_bias, c.D, c.A,
                     c.conv_state_in, c.ssm_state_in, y, c.conv_state_out, c.ssm_state_out, c.workspace);
  return hipGetLastError();
}

}  // namespace

#ifndef MSCAN_FWD_KIND
#define MSCAN_FWD_KIND 1
#endif
#ifndef MSCAN_ROW_FOR_N16
#define MSCAN_ROW_FOR_N16 1
#endif
#ifndef MSCAN_QUAD_MIN_WAVES
#define MSCAN_QUAD_MIN_WAVES 2048
#endif
#ifndef MSCAN_QUAD_TARGET_WAVES
#define MSCAN_QUAD_TARGET_WAVES 3072
#endif
#ifndef MSCAN_ROW_MIN_WAVES
#define MSCAN_ROW_MIN_WAVES 2048  // fewer waves per chunk: the quad kernel is used
#endif
#ifndef MSCAN_ROW_TARGET_WAVES
#define MSCAN_ROW_TARGET_WAVES 3072
#endif

namespace {
FwdPlan plan_fwd_kind(int32_t batch, int32_t seqlen, int32_t d_inner, int32_t d_state, int32_t io_dtype,
                      int forced) {
  FwdPlan p;
  p.kind = forced >= 0 ? forced : MSCAN_FWD_KIND;
  if (p.kind == kFwdQuad || p.kind == kFwdRow) {
    // d_state 16 with enough channels for ~2 waves per SIMD at 16 lanes per
    // channel: the row kernel, sequence unsplit. Otherwise the quad kernel
    // (4 lanes per channel), splitting the sequence until the launch has
    // about MSCAN_QUAD_TARGET_WAVES waves (twice that where the chunks stay
    // 1024 steps or longer): the split costs a second sweep of the
    // exponentials over all but the last chunk, and for long sequences a
    // finer split of the quad kernel measured faster than a coarse split of
    // the row kernel.
    // Sequences of up to 1024 steps also take the row kernel at d_state 16:
    // its four times the quad kernel's waves need fewer (or no) chunks, and
    // short chunks cost the quad kernel its pipeline fill (measured at
    // batch 1-4, d_inner 768-2560: at 512 steps the row kernel took 0.66-1.09
    // of the quad kernel's time, at 2048 0.75-1.17, at 8192 and more mostly
    // longer; the 2 x 64 x 128 prefill 6.5 against 11.1 us).
    const int64_t row_waves = static_cast<int64_t>(batch) * ((d_inner + 15) / 16) * 4;
    if (forced < 0) {
      const bool short_seq = seqlen <= 1024;
      p.kind = (d_state == 16 && MSCAN_ROW_FOR_N16 && (row_waves >= MSCAN_ROW_MIN_WAVES || short_seq)) ? kFwdRow
                                                                                                      : kFwdQuad;
    }
    const int64_t waves = p.kind == kFwdRow ? row_waves : static_cast<int64_t>(batch) * ((d_inner + 63) / 64) * 4;
    const int64_t target = p.kind == kFwdRow ? MSCAN_ROW_TARGET_WAVES : MSCAN_QUAD_TARGET_WAVES;
    const int64_t max_nc = seqlen / kMinChunk;
    auto chunks_for = [&](int64_t t) {
      int64_t c = waves < MSCAN_QUAD_MIN_WAVES ? (t + waves - 1) / waves : 1;
      return c > max_nc ? max_nc : c;
    };
    int64_t nc = chunks_for(target);
    // The quad kernel's chunks already 1024 steps or longer at that target:
    // twice the waves cost them little per-chunk overhead and hide more
    // latency (the long prefill, 1 x 65536 x 1536: 6144 waves measured faster
    // than 4032, 8064 or 12000; shorter chunks do best at ~3072 waves).
    if (p.kind == kFwdQuad && nc >= 1 && seqlen / (nc > 0 ? nc : 1) >= 1024) nc = chunks_for(2 * target);
    if (nc < 1) nc = 1;
    int64_t len = (seqlen + nc - 1) / nc;
    len = (len + 15) / 16 * 16;
    nc = (seqlen + len - 1) / len;
    p.n_chunks = static_cast<int32_t>(nc);
    p.chunk_len = nc > 1 ? static_cast<int32_t>(len) : seqlen;
    p.ws_floats = quad_ws_layout(batch, d_inner, d_state, p.n_chunks).total;
    return p;
  }
  const int64_t waves_per_chunk = static_cast<int64_t>(batch) * ((d_inner + kWave - 1) / kWave);
  int64_t nc = (kTargetWaves + waves_per_chunk - 1) / waves_per_chunk;
  const int64_t max_nc = seqlen / kMinChunk;  // every chunk at least kMinChunk long
  if (nc > max_nc) nc = max_nc;
  if (nc < 1) nc = 1;
  int64_t len = (seqlen + nc - 1) / nc;
  len = (len + 7) / 8 * 8;
  nc = (seqlen + len - 1) / len;
  if (nc <= 1) {
    p.n_chunks = 1;
    p.chunk_len = seqlen;
  } else {
    p.n_chunks = static_cast<int32_t>(nc);
    p.chunk_len = static_cast<int32_t>(len);
  }
  p.ws_floats = ws_layout(batch, seqlen, d_inner, d_state, p.n_chunks, io_dtype == 1).total;
  return p;
}
}  // namespace

FwdPlan plan_fwd(int32_t batch, int32_t seqlen, int32_t d_inner, int32_t d_state, int32_t io_dtype,
                 int32_t forced_kind) {
  if (forced_kind == kFwdRow && d_state != 16) forced_kind = -1;  // the row kernel serves d_state 16 only
  return plan_fwd_kind(batch, seqlen, d_inner, d_state, io_dtype, forced_kind);
}

FwdPlan plan_fwd_row(int32_t batch, int32_t seqlen, int32_t d_inner, int32_t io_dtype) {
  return plan_fwd_kind(batch, seqlen, d_inner, 16, io_dtype, kFwdRow);
}

hipError_t launch_fwd(const FwdCall& c, const FwdPlan& p) {
  if (c.dt_low && p.kind != kFwdRow) return hipErrorInvalidValue;  // dt_proj inside: row kernel only
  if (p.kind == kFwdRow) return launch_fwd_row(c, p);
  if (p.kind == kFwdQuad) return launch_fwd_quad(c, p);
  if (c.io_dtype == 0) {
    return c.d_state == 16 ? launch_typed<0, 16>(c, p) : launch_typed<0, 8>(c, p);
  }
  return c.d_state == 16 ? launch_typed<1, 16>(c, p) : launch_typed<1, 8>(c, p);
}

}  // namespace mscan
