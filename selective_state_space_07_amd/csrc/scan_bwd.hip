// Backward of the prefill for gfx950 (d_state = 16): gradients of
// L = sum(y * dy) with respect to x, dt, z, B, C and the parameters, for the
// operation of calm-mamba 0.1.4 PKG-INFO, "Mamba operator", steps 2, 4, 5, 6
// (the page's kernels recompute the forward in their backward; so does this).
//
// Work layout: sixteen lanes per channel as in the prefill (lane n keeps state
// n; a 256-thread workgroup serves 16 channels of one batch row).
//  1. checkpoint pass: the prefill's sixteen-lane kernel (scan_fwd_row.hip)
//     in its checkpoint-only form runs the forward recurrence over the whole
//     sequence and saves h before every stage of 16 timesteps
//     ([batch][stages][d_inner][16] float32); no outputs. Skipped when the
//     caller passes the forward's own checkpoints.
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
// The reverse kernel loads the next stage's inputs while the current one
// runs, through branch-free buffer loads (out-of-range offsets read zeros), so
// the loads stay in flight across the stage; with loads under branches the
// compiler waits for them at once and every stage pays the memory latency.
// Gradients with respect to the initial states are not produced.
#include "scan_device.h"
#include "scan_fwd_common.h"
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
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, true));
}
__device__ __forceinline__ float row_sum(float v) {
  v += dpp<0x128>(v);
  v += dpp<0x124>(v);
  v += dpp<0x122>(v);
  v += dpp<0x121>(v);
  return v;
}
// Sixteen row sums at once, scattered: every lane of a 16-lane row holds
// v[0..15]; lane n of the row returns the sum over the row's lanes of v[n].
// A butterfly over the lane-index bits 3, 2, 1, 0 (partners n^15, n^7, n^2,
// n^1: row mirror, half-row mirror, quad swaps): at each level a lane keeps
// the half of its values whose index agrees with its own bit and adds the
// partner's matching half. 15 DPP adds instead of 16 x 4.
__device__ __forceinline__ float row_scatter16(const float (&v)[16], int n) {
  const bool b3 = (n & 8) != 0, b2 = (n & 4) != 0, b1 = (n & 2) != 0, b0 = (n & 1) != 0;
  float r8[8], r4[4], r2[2];
#pragma unroll
  for (int i = 0; i < 8; ++i) r8[i] = (b3 ? v[8 + i] : v[i]) + dpp<0x140>(b3 ? v[i] : v[8 + i]);
#pragma unroll
  for (int i = 0; i < 4; ++i) r4[i] = (b2 ? r8[4 + i] : r8[i]) + dpp<0x141>(b2 ? r8[i] : r8[4 + i]);
#pragma unroll
  for (int i = 0; i < 2; ++i) r2[i] = (b1 ? r4[2 + i] : r4[i]) + dpp<0x4E>(b1 ? r4[i] : r4[2 + i]);
  return (b0 ? r2[1] : r2[0]) + dpp<0xB1>(b0 ? r2[0] : r2[1]);
}

// Workgroup blockIdx.x serves channel group g = blockIdx.x % groups of batch
// row b = blockIdx.x / groups (one grid dimension, so any batch fits).
struct Chan {
  int32_t b, g, d;
  bool active;
};
__device__ __forceinline__ Chan channel(int32_t d_inner, int32_t groups, int tid) {
  // Workgroups are dispatched to the 8 XCDs round-robin by linear id, and each
  // XCD has its own L2. Consecutive channel groups share the cache lines of
  // x, dt, z, dy and of the gradients, and one batch row shares B and C, so
  // each XCD is given a contiguous range of (batch row, channel group) ids.
  const int32_t nb = static_cast<int32_t>(gridDim.x), p = static_cast<int32_t>(blockIdx.x);
  const int32_t q = nb >> 3, r = nb & 7, x = p & 7, i = p >> 3;
  const int32_t blk = x * q + min(x, r) + i;
  const int32_t b = blk / groups, g = blk - b * groups;
  const int32_t d_raw = g * kCPB + (tid >> 4);
  return Chan{b, g, d_raw < d_inner ? d_raw : d_inner - 1, d_raw < d_inner};
}

// Per-element forward terms. Past the end of the sequence delta is set to 0,
// which makes the step the identity (decay 1, input 0): a ragged last stage
// runs the same code as a full one, its extra steps change no state and
// contribute nothing to any gradient (their dy, B and C are zero too).
struct Elem {
  float u, su, xc, v, delta, dx;  // su = sigmoid(u), xc = u su, dx = delta xc
};
__device__ __forceinline__ Elem make_elem(const float (&xw)[4], float dtv, const float (&w)[4], float cb,
                                          float dtb, bool valid) {
  Elem e;
  float u = cb;
#pragma unroll
  for (int k = 0; k < 4; ++k) u = fmaf(w[k], xw[k], u);
  e.u = u;
  e.su = sigmoid_hw(u);
  e.xc = u * e.su;
  e.v = dtv + dtb;
  e.delta = valid ? softplus(e.v) : 0.0f;
  e.dx = e.delta * e.xc;
  return e;
}

// Four consecutive timesteps j0 .. j0+3 of state n from a transposed [n][j] tile.
__device__ __forceinline__ float4 tile4(const float* row, int j0) {
  return *reinterpret_cast<const float4*>(row + j0);
}
__device__ __forceinline__ float pick(const float4& q, int k) {
  return k == 0 ? q.x : (k == 1 ? q.y : (k == 2 ? q.z : q.w));
}

constexpr int kRow = kStage + 4;  // padded row of a transposed [n][j] tile

// Lane addressing: every access is a buffer descriptor on a wave-uniform base
// (computed per stage in scalar registers) plus a per-lane 32-bit byte offset
// fixed for the whole kernel, so no per-access 64-bit vector address math.
template <typename T>
__device__ __forceinline__ T* shift(T* base, int64_t elems) {  // may point before the array; not dereferenced there
  return reinterpret_cast<T*>(reinterpret_cast<uintptr_t>(base) + elems * static_cast<int64_t>(sizeof(T)));
}
struct LaneOff {
  uint32_t e;     // (own timestep row n, channel d) in io elements, as bytes
  uint32_t tile;  // B / C tile element (row tj, state n), as bytes
  uint32_t ck;    // checkpoint (channel d, state n), as bytes
};
template <int IO>
__device__ __forceinline__ LaneOff lane_offsets(int32_t D, int32_t d, int n, int tj) {
  const uint32_t es = sizeof(typename Io<IO>::T);
  return LaneOff{(static_cast<uint32_t>(n) * D + d) * es, (static_cast<uint32_t>(tj) * kN + n) * es,
                 (static_cast<uint32_t>(d) * kN + n) * 4u};
}

// Inputs of one stage for one thread: its own timestep's dt, z, dy and the
// stage's checkpoint, and its element (timestep tid / 16, state tid % 16) of
// the stage's B / C tile. Its x row is fetched two stages ahead on its own;
// the rest of the conv window comes from neighbouring lanes.
struct StageIn {
  uint32_t dt, z, dy, hck, b, c;  // raw bits as loaded (bfloat16 in the low half)
};
// A raw buffer descriptor from a wave-uniform base (the base may lie before
// the array when the first bytes are never accessed). Offsets at or past
// kWin read 0 and write nothing, which makes every load below branch-free:
// a lane with nothing to load passes kOff, so the value waits in its register
// until it is used (a load under a branch is waited for at the branch's end).
constexpr uint32_t kWin = 0x7FFFFFF0u;
constexpr uint32_t kOff = 0xFFFFFFFFu;
template <typename T>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc_at(T* base, int64_t elems) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(static_cast<const void*>(shift(base, elems))), 0,
                                           static_cast<int32_t>(kWin), 0x00020000);
}
template <int IO>
__device__ __forceinline__ uint32_t ldr(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  if constexpr (IO == 0) {
    return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
  } else {
    return __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0);
  }
}
template <int IO>
__device__ __forceinline__ float cvt(uint32_t v) {
  return IO == 0 ? __builtin_bit_cast(float, v) : __builtin_bit_cast(float, v << 16);
}
__device__ __forceinline__ void st_f32(__amdgpu_buffer_rsrc_t r, uint32_t off, float v) {
  __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), r, off, 0, 0);
}

template <int IO>
__device__ __forceinline__ void fetch_stage(StageIn& in, int32_t s, int32_t seqlen, int32_t D, int32_t stages,
                                            int32_t b, int n, int tj, const LaneOff& lo,
                                            const typename Io<IO>::T* dt,
                                            const typename Io<IO>::T* z, const typename Io<IO>::T* dy,
                                            const typename Io<IO>::T* Bm, const typename Io<IO>::T* Cm,
                                            const float* ckpt) {
  // s outside [0, stages) loads nothing (all offsets kOff), without a branch.
  // The B / C tile is loaded first: it is needed first (staged into LDS at
  // the end of the current stage), and loads complete in issue order.
  const bool sv = s >= 0 && s < stages;
  const int32_t sc = sv ? s : 0;
  const int64_t row0 = static_cast<int64_t>(b) * seqlen;
  const int32_t ts = sc * kStage, t = ts + n;
  const uint32_t ot = (sv && ts + tj < seqlen) ? lo.tile : kOff;
  in.b = ldr<IO>(rsrc_at(Bm, (row0 + ts) * kN), ot);
  in.c = ldr<IO>(rsrc_at(Cm, (row0 + ts) * kN), ot);
  in.hck = __builtin_amdgcn_raw_buffer_load_b32(rsrc_at(ckpt, (static_cast<int64_t>(b) * stages + sc) * D * kN),
                                                sv ? lo.ck : kOff, 0, 0);
  const bool tv = sv && t < seqlen;
  const int64_t rs = (row0 + ts) * D;
  const uint32_t oe = tv ? lo.e : kOff;
  in.dt = ldr<IO>(rsrc_at(dt, rs), oe);
  in.z = ldr<IO>(rsrc_at(z, rs), oe);
  in.dy = ldr<IO>(rsrc_at(dy, rs), oe);
}

// The conv window x[t-3 .. t] of the lane's timestep t = ts + n from the own
// row x[t] alone: the earlier rows are the same row's values in lanes n-1 ..
// n-3 (row shifts), and for the first lanes the last three rows of the stage
// before, xlast = x[ts-3 .. ts-1] (the conv history in stage 0).
template <int K>
__device__ __forceinline__ float shr(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x110 + K, 0xF, 0xF, true));
}
__device__ __forceinline__ void window_shift(float (&xw)[4], float x0, const float (&xlast)[3], int n) {
  const float m1 = shr<1>(x0), m2 = shr<2>(x0), m3 = shr<3>(x0);
  xw[3] = x0;
  xw[2] = n >= 1 ? m1 : xlast[2];
  xw[1] = n >= 2 ? m2 : (n == 1 ? xlast[2] : xlast[1]);
  xw[0] = n >= 3 ? m3 : (n == 2 ? xlast[2] : (n == 1 ? xlast[1] : xlast[0]));
}

// The own row x[16 s + n] of stage s (0 outside the sequence), branch-free.
template <int IO>
__device__ __forceinline__ uint32_t load_xrow(const typename Io<IO>::T* x, int32_t s, int32_t seqlen, int32_t D,
                                              int32_t stages, int32_t b, int n, const LaneOff& lo) {
  const bool sv = s >= 0 && s < stages;
  const int32_t ts = (sv ? s : 0) * kStage;
  const bool tv = sv && ts + n < seqlen;
  return ldr<IO>(rsrc_at(x, (static_cast<int64_t>(b) * seqlen + ts) * D), tv ? lo.e : kOff);
}

// Backward over the stages in reverse. Per stage: barrier; prefetch the
// earlier stage's inputs; recompute the forward from the checkpoint; adjoint
// through the 16 steps (dB / dC contributions into LDS); element backward;
// barrier; sum the dB / dC contributions over the workgroup's channels and
// stage the earlier stage's B / C tile (double-buffered), so two barriers per
// stage.
template <int IO>
__global__ __launch_bounds__(kThreads) void bwd_kernel(
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
  __shared__ __align__(16) float bc[2][2][kN][kRow];   // [B | C][buffer][n][timestep]
  // dB / dC contributions, [channel][timestep * 16 + n]; the channel stride
  // (272 words, 16 mod 32) keeps a half-wave's writes (two channels, one
  // timestep) on distinct banks, and rows of 16 make a half-wave's reads (two
  // timesteps of one channel) one contiguous 32-word span
  __shared__ float part[2][kCPB][kStage * kN + 16];
  const int tid = threadIdx.x, n = tid & (kN - 1), cl = tid >> 4, tj = tid >> 4;
  const int32_t D = d_inner;
  const Chan c = channel(D, groups, tid);
  const int32_t d = c.d, b = c.b;
  const float w[4] = {conv_w[d * 4], conv_w[d * 4 + 1], conv_w[d * 4 + 2], conv_w[d * 4 + 3]};
  const float cb = conv_b[d], dtb = dt_bias[d], Dd = Dskip[d];
  const float An = A[d * kN + n], A2 = An * kLog2e;
  const float* hist = conv0 ? conv0 + (static_cast<size_t>(b) * D + d) * 3 : nullptr;

  float dh = 0.0f;
  float g_dA = 0.0f, g_dD = 0.0f, g_dtb = 0.0f, g_cb = 0.0f, g_cw[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  float carry0 = 0.0f, carry1 = 0.0f, carry2 = 0.0f;  // du of the first three steps of the later stage

  const float hv[3] = {hist ? hist[0] : 0.0f, hist ? hist[1] : 0.0f, hist ? hist[2] : 0.0f};
  StageIn in;
  const LaneOff lo = lane_offsets<IO>(D, d, n, tj);
  fetch_stage<IO>(in, stages - 1, seqlen, D, stages, b, n, tj, lo, dt, z, dy, Bm, Cm, ckpt);
  // the own x row is fetched two stages ahead: stage s's window needs the
  // last rows of stage s - 1, which are then already loaded
  uint32_t xcur = load_xrow<IO>(x, stages - 1, seqlen, D, stages, b, n, lo);
  uint32_t xnext = load_xrow<IO>(x, stages - 2, seqlen, D, stages, b, n, lo);
  bc[0][(stages - 1) & 1][n][tj] = cvt<IO>(in.b);
  bc[1][(stages - 1) & 1][n][tj] = cvt<IO>(in.c);

  for (int32_t s = stages - 1; s >= 0; --s) {
    const int32_t ts = s * kStage;
    const int nv = min(kStage, seqlen - ts);  // valid steps of this stage (wave-uniform)
    __syncthreads();
    __builtin_amdgcn_s_setprio(1);  // the fetches and the element terms of the stage
    const StageIn cur = in;
    // prefetch the earlier stage (nothing before the first)
    fetch_stage<IO>(in, s - 1, seqlen, D, stages, b, n, tj, lo, dt, z, dy, Bm, Cm, ckpt);
    const float x0 = cvt<IO>(xcur), xe = cvt<IO>(xnext);  // own rows of stages s and s - 1
    xcur = xnext;
    xnext = load_xrow<IO>(x, s - 2, seqlen, D, stages, b, n, lo);
    const int64_t rs = (static_cast<int64_t>(b) * seqlen + ts) * D;  // element row ts of this batch row
    const auto dzr = rsrc_at(dz, rs), ddtr = rsrc_at(ddt, rs), dxr = rsrc_at(dx, rs);
    const bool valid = n < nv;
    float xw[4];
    {
      const float xlast[3] = {s > 0 ? bcast<13>(xe) : hv[0], s > 0 ? bcast<14>(xe) : hv[1],
                              s > 0 ? bcast<15>(xe) : hv[2]};
      window_shift(xw, x0, xlast, n);
    }
    const Elem e = make_elem(xw, cvt<IO>(cur.dt), w, cb, dtb, valid);
    const float zt = cvt<IO>(cur.z), dyt = c.active ? cvt<IO>(cur.dy) : 0.0f;
    const float hprev = __builtin_bit_cast(float, cur.hck);
    const float sz = sigmoid_hw(zt);
    const float dyr = dyt * (zt * sz);  // dL/d(pre-gate y); 0 past the end
    const float* brow = bc[0][s & 1][n];
    const float* crow = bc[1][s & 1][n];

    // forward recompute of the stage from its checkpoint. Wave priorities
    // (s_setprio): the two dependent chains (this recompute and the adjoint)
    // first, the element backward second, the fetches and element terms
    // third, the barriers and dB / dC sums last (measured: ~680 -> ~626-640 us,
    // results bit for bit the same).
    float H[kStage], yv[kStage];
    float h = hprev;
    __builtin_amdgcn_s_setprio(3);
#pragma unroll
    for (int j4 = 0; j4 < kStage; j4 += 4) {
      const float4 b4 = tile4(brow, j4), c4 = tile4(crow, j4);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int j = j4 + k;
        const float dj = bcast_j(e.delta, j), dxj = bcast_j(e.dx, j);
        const float aj = exp2_hw(dj * A2);
        h = fmaf(aj, h, dxj * pick(b4, k));
        H[j] = h;
        yv[j] = pick(c4, k) * h;  // this state's share of step j's readout
      }
    }
    const float yraw = fmaf(Dd, e.xc, row_scatter16(yv, n));  // readout of the own step
    // adjoint through the 16 steps, newest first; the decays are recomputed
    // (an opaque copy of A log2(e) keeps the compiler from reusing, and so
    // keeping live, the sixteen of the recompute above)
    float A2r = A2;
    asm volatile("" : "+v"(A2r));
    float Tv[kStage], Sv[kStage];
#pragma unroll
    for (int j4 = kStage - 4; j4 >= 0; j4 -= 4) {
      const float4 b4 = tile4(brow, j4), c4 = tile4(crow, j4);
#pragma unroll
      for (int k = 3; k >= 0; --k) {
        const int j = j4 + k;
        const float dyrj = bcast_j(dyr, j), dxj = bcast_j(e.dx, j), dj = bcast_j(e.delta, j);
        dh = fmaf(pick(c4, k), dyrj, dh);
        part[1][cl][j * kN + n] = H[j] * dyrj;        // dC contribution
        const float hp = j > 0 ? H[j - 1] : hprev;
        const float aj = exp2_hw(dj * A2r);
        const float q = dh * (aj * hp);
        g_dA = fmaf(q, dj, g_dA);
        Tv[j] = q * An;                               // share of step j's ddelta (decay term)
        Sv[j] = dh * pick(b4, k);                     // share of sum_n dh B (input term per unit delta xc)
        part[0][cl][j * kN + n] = dh * dxj;           // dB contribution
        dh *= aj;
      }
    }
    __builtin_amdgcn_s_setprio(2);
    const float T_me = row_scatter16(Tv, n), S_me = row_scatter16(Sv, n);
    // element backward of the own timestep
    float du = 0.0f;
    if (valid) {
      if (c.active) buf_store<IO>(dyt * yraw * sz * (1.0f + zt * (1.0f - sz)), dzr, lo.e, 0);
      g_dD = fmaf(dyr, e.xc, g_dD);
      const float dxc = fmaf(dyr, Dd, e.delta * S_me);
      const float ddelta = fmaf(e.xc, S_me, T_me);
      const float dv = ddelta * sigmoid_hw(e.v);
      if (c.active) buf_store<IO>(dv, ddtr, lo.e, 0);
      g_dtb += dv;
      du = dxc * e.su * (1.0f + e.u * (1.0f - e.su));
      g_cb += du;
#pragma unroll
      for (int k = 0; k < 4; ++k) g_cw[k] = fmaf(du, xw[k], g_cw[k]);
    }
    // dx[t] = w3 du[t] + w2 du[t+1] + w1 du[t+2] + w0 du[t+3]
    const float du1 = __shfl_down(du, 1, kN), du2 = __shfl_down(du, 2, kN), du3 = __shfl_down(du, 3, kN);
    const float n1 = n + 1 < kN ? du1 : carry0;
    const float n2 = n + 2 < kN ? du2 : (n == 14 ? carry0 : carry1);
    const float n3 = n + 3 < kN ? du3 : (n == 13 ? carry0 : (n == 14 ? carry1 : carry2));
    if (valid && c.active) {
      const float gx = fmaf(w[0], n3, fmaf(w[1], n2, fmaf(w[2], n1, w[3] * du)));
      buf_store<IO>(gx, dxr, lo.e, 0);
    }
    carry0 = bcast<0>(du);
    carry1 = bcast<1>(du);
    carry2 = bcast<2>(du);
    __builtin_amdgcn_s_setprio(0);
    __syncthreads();
    // dB / dC of the stage summed over the workgroup's channels, in channel order
    if (tj < nv) {
      float sb = 0.0f, sc = 0.0f;
#pragma unroll
      for (int k = 0; k < kCPB; ++k) {  // channels past d_inner hold zeros
        sb += part[0][k][tj * kN + n];
        sc += part[1][k][tj * kN + n];
      }
      const int64_t o = ((static_cast<int64_t>(b) * groups + c.g) * seqlen + ts) * kN;
      st_f32(rsrc_at(dBpart, o), (static_cast<uint32_t>(tj) * kN + n) * 4u, sb);
      st_f32(rsrc_at(dCpart, o), (static_cast<uint32_t>(tj) * kN + n) * 4u, sc);
    }
    // stage the earlier stage's B / C tile; unconditional (after stage 0 it
    // fills the idle buffer with zeros), so no branch splits the stage's code
    bc[0][(s - 1) & 1][n][tj] = cvt<IO>(in.b);
    bc[1][(s - 1) & 1][n][tj] = cvt<IO>(in.c);
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

// 3a. dB[b][t][n] = sum over workgroups of the partials. Four lanes of a quad
// share four consecutive n of one (b, t) (16-byte loads from the workspace,
// which is 256-byte aligned) and each sums a contiguous quarter of the
// workgroups in order; the quarters are then added as (q0 + q1) + (q2 + q3),
// a fixed order, so the result is deterministic. Four lanes per output keep
// enough loads in flight. dB and dC are written with 4-byte stores (no
// alignment assumed).
__device__ __forceinline__ float quad_sum(float v) {
  v += dpp<0xB1>(v);  // quad_perm [1,0,3,2]: q0+q1 | q2+q3
  return v + dpp<0x4E>(v);  // quad_perm [2,3,0,1]: (q0+q1) + (q2+q3), same in every lane
}
__global__ __launch_bounds__(kThreads) void bwd_reduce_bc_kernel(int64_t total4, int32_t seqlen, int32_t groups,
                                                                 const float* __restrict__ pB,
                                                                 const float* __restrict__ pC, float* __restrict__ dB,
                                                                 float* __restrict__ dC) {
  const int64_t gid = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  const int64_t i = gid >> 2;  // (b, t, n / 4); the grid covers whole quads
  const int q = static_cast<int>(gid & 3);
  const bool live = i < total4;
  const int64_t ii = live ? i : 0;
  const int64_t per_b4 = static_cast<int64_t>(seqlen) * (kN / 4);
  const int64_t b = ii / per_b4, r = ii - b * per_b4;
  const int32_t span = (groups + 3) >> 2, g0 = min(groups, q * span), g1 = min(groups, g0 + span);
  const float4* qB = reinterpret_cast<const float4*>(pB) + b * groups * per_b4 + r;
  const float4* qC = reinterpret_cast<const float4*>(pC) + b * groups * per_b4 + r;
  float4 sb = {0.0f, 0.0f, 0.0f, 0.0f}, sc = sb;
#pragma unroll 8
  for (int32_t g = g0; g < g1; ++g) {
    const float4 vb = qB[g * per_b4], vc = qC[g * per_b4];
    sb.x += vb.x; sb.y += vb.y; sb.z += vb.z; sb.w += vb.w;
    sc.x += vc.x; sc.y += vc.y; sc.z += vc.z; sc.w += vc.w;
  }
  sb.x = quad_sum(sb.x); sb.y = quad_sum(sb.y); sb.z = quad_sum(sb.z); sb.w = quad_sum(sb.w);
  sc.x = quad_sum(sc.x); sc.y = quad_sum(sc.y); sc.z = quad_sum(sc.z); sc.w = quad_sum(sc.w);
  if (live && q == 0) {
    float* ob = dB + i * 4;
    float* oc = dC + i * 4;
    ob[0] = sb.x; ob[1] = sb.y; ob[2] = sb.z; ob[3] = sb.w;
    oc[0] = sc.x; oc[1] = sc.y; oc[2] = sc.z; oc[3] = sc.w;
  }
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
  const BwdWs w = bwd_ws_layout(c.batch, c.seqlen, c.d_inner, c.ckpt == nullptr);
  const int32_t stages = (c.seqlen + kStage - 1) / kStage;
  const int32_t groups = (c.d_inner + kCPB - 1) / kCPB;
  float* pB = c.workspace + w.dBpart;
  float* pC = c.workspace + w.dCpart;
  float* pg = c.workspace + w.pgrad;
  const dim3 grid(static_cast<unsigned>(groups) * static_cast<unsigned>(c.batch));
  hipError_t e;
  const float* ckpt = c.ckpt;
  if (!ckpt) {  // recompute the forward's states every 16 steps
    float* own = c.workspace + w.ckpt;
    FwdCall f{};
    f.batch = c.batch;
    f.seqlen = c.seqlen;
    f.d_inner = c.d_inner;
    f.d_state = kN;
    f.io_dtype = IO;
    f.x = c.x;
    f.dt = c.dt;
    f.B = c.B;  // z, C and y take no part in the checkpoint pass
    f.conv_w = c.conv_w;
    f.conv_b = c.conv_b;
    f.dt_bias = c.dt_bias;
    f.A = c.A;
    f.conv_state_in = c.conv_state_in;
    f.ssm_state_in = c.ssm_state_in;
    f.stream = c.stream;
    f.ckpt = own;
    f.ckpt_only = true;
    f.bc_stride = kN;
    FwdPlan p{};
    p.kind = kFwdRow;
    p.n_chunks = 1;
    p.chunk_len = c.seqlen;
    e = launch_fwd_row(f, p);
    if (e != hipSuccess) return e;
    ckpt = own;
  }
  hipLaunchKernelGGL((bwd_kernel<IO>), grid, dim3(kThreads), 0, c.stream, c.seqlen, c.d_inner, stages, groups,
                     static_cast<const T*>(c.x), static_cast<const T*>(c.dt), static_cast<const T*>(c.z),
                     static_cast<const T*>(c.B), static_cast<const T*>(c.C), c.conv_w, c.conv_b, c.dt_bias, c.D, c.A,
                     c.conv_state_in, ckpt, static_cast<const T*>(c.dy), static_cast<T*>(c.dx),
                     static_cast<T*>(c.ddt), static_cast<T*>(c.dz), pB, pC, pg);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t total4 = static_cast<int64_t>(c.batch) * c.seqlen * (kN / 4);
  hipLaunchKernelGGL(bwd_reduce_bc_kernel, dim3(static_cast<unsigned>((4 * total4 + kThreads - 1) / kThreads)),
                     dim3(kThreads), 0, c.stream, total4, c.seqlen, groups, pB, pC, c.dB, c.dC);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int32_t np = c.d_inner * (kN + 7);
  hipLaunchKernelGGL(bwd_reduce_params_kernel, dim3(static_cast<unsigned>((np + kThreads - 1) / kThreads)),
                     dim3(kThreads), 0, c.stream, c.batch, c.d_inner, pg, c.dconv_w, c.dconv_b, c.ddt_bias, c.dD,
                     c.dA);
  return hipGetLastError();
}

}  // namespace

size_t ckpt_floats(int32_t batch, int32_t seqlen, int32_t d_inner) {
  const size_t stages = (static_cast<size_t>(seqlen) + kStage - 1) / kStage;
  return static_cast<size_t>(batch) * d_inner * stages * kN;
}

BwdWs bwd_ws_layout(int32_t batch, int32_t seqlen, int32_t d_inner, bool own_ckpt) {
  BwdWs w{};
  const size_t groups = (static_cast<size_t>(d_inner) + kCPB - 1) / kCPB;
  w.ckpt = 0;
  w.dBpart = w.ckpt + (own_ckpt ? ckpt_floats(batch, seqlen, d_inner) : 0);
  w.dCpart = w.dBpart + static_cast<size_t>(batch) * groups * seqlen * kN;
  w.pgrad = w.dCpart + static_cast<size_t>(batch) * groups * seqlen * kN;
  w.total = w.pgrad + static_cast<size_t>(batch) * d_inner * kPG;
  return w;
}

hipError_t launch_bwd(const BwdCall& c) {
  return c.io_dtype == 0 ? launch_typed<0>(c) : launch_typed<1>(c);
}

}  // namespace mscan
