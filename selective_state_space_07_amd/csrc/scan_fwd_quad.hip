// Prefill kernels of libmamba_scan for gfx950: four lanes per channel.
//
// Computes, for every batch row b and channel d (calm-mamba 0.1.4 PKG-INFO,
// "Mamba operator", steps 2, 4, 5, 6): the causal depthwise conv (4 taps) +
// SiLU, delta = softplus(dt + dt_bias), the recurrence
// h[n] = exp(delta*A[n])*h[n] + delta*B[n]*xc with readout C.h + D*xc, and the
// SiLU(z) gate; plus the final conv and SSM states.
//
// Work layout. A channel is served by a quad of 4 lanes; lane g of the quad
// keeps the states n = g*N/4 .. g*N/4 + N/4 - 1 in VGPRs, so a wave covers 16
// channels and the launch has four times as many lanes as channels (the
// channels alone cannot fill 1024 SIMDs on the workloads of interest).
// Time advances in blocks of 4 timesteps: lane g computes the per-element
// terms (conv, SiLU, softplus, gate) of timestep 4k+g only, and the quad
// shares delta and delta*xc with DPP quad broadcasts, so that per-element work
// is not repeated. Each lane accumulates the readout over its own states for
// the 4 timesteps of a block; a DPP transposed reduction then leaves in lane g
// the full sum for timestep 4k+g, which lane g gates and stores.
// B and C rows (shared by all channels of a batch row) are staged per 16
// timesteps in LDS by the 256-thread workgroup and read back as 16-byte
// broadcast reads.
//
// The sequence can also be split into chunks (for batch rows with few
// channels and long sequences). The recurrence is affine in h, so a chunk acts
// on the state as h -> P*h + S with P[n] = exp(A[n] * sum of its deltas) and S
// its end state from zero; these pairs compose associatively (not
// commutatively). The summary pass computes (sum delta, S) for every chunk but
// the last; the final pass folds the summaries of all earlier chunks into its
// carry-in and then runs its chunk.
#include <type_traits>

#include "scan_device.h"
#include "scan_fwd_common.h"
#include "scan_internal.h"

namespace mscan {

namespace {

// Occupancy request: the compiler then fits the final pass in 127 VGPRs and
// the summary pass in 100, four waves per SIMD each, without spilling (a
// request of 4 leaves a small scratch spill in the final pass).
#ifndef MSCAN_QUAD_WAVES_PER_EU
#define MSCAN_QUAD_WAVES_PER_EU 5
#endif

constexpr int kThreads = 256;  // 4 waves, 64 channels
constexpr int kG = 4;          // lanes per channel
constexpr int kStage = 16;     // timesteps of B/C staged in LDS at a time

enum Pass { kSummary = 0, kFinal = 1 };

// Broadcast the value held by lane J of each quad to the whole quad.
template <int J>
__device__ __forceinline__ float quad_bcast(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), J * 0x55, 0xF, 0xF, true));
}
__device__ __forceinline__ float quad_bcast_j(float v, int j) {
  switch (j) {
    case 0: return quad_bcast<0>(v);
    case 1: return quad_bcast<1>(v);
    case 2: return quad_bcast<2>(v);
    default: return quad_bcast<3>(v);
  }
}
// Value of the lane whose index differs in bit 0 (xor1) or bit 1 (xor2).
__device__ __forceinline__ float quad_xor1(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, true));  // [1,0,3,2]
}
__device__ __forceinline__ float quad_xor2(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, true));  // [2,3,0,1]
}

// In: p[j] = this lane's partial sum for timestep j of the block (j = 0..3).
// Out: the sum over the quad of p[g], g = this lane's index in the quad.
// Two butterfly stages; each lane keeps half of what it holds and sends the
// other half to its partner.
__device__ __forceinline__ float quad_transpose_sum(const float (&p)[4], bool bit1, bool bit0) {
  const float keep0 = bit1 ? p[2] : p[0];
  const float send0 = bit1 ? p[0] : p[2];
  const float keep1 = bit1 ? p[3] : p[1];
  const float send1 = bit1 ? p[1] : p[3];
  const float q0 = keep0 + quad_xor2(send0);
  const float q1 = keep1 + quad_xor2(send1);
  const float keep = bit0 ? q1 : q0;
  const float send = bit0 ? q0 : q1;
  return keep + quad_xor1(send);
}

// Per-stage tiles in LDS, double-buffered, all float32:
//   bc  [buffer][B or C][timestep in stage][n]
//   xt  [buffer][row][channel]  x rows ts-3 .. ts+15 (conv windows of the stage)
//   dtt, zt [buffer][row][channel]  rows ts .. ts+15
// A row of 64 channels is padded to 80 floats so that the four rows a quad
// reads at once fall in distinct LDS banks.
constexpr int kRowPad = 80;
template <int N>
struct alignas(16) Tiles {
  float bc[2][2][kStage][N];
  float xt[2][kStage + 3][kRowPad];
  float dtt[2][kStage][kRowPad];
  float zt[2][kStage][kRowPad];
  int32_t sq[2][kStage + 4];  // document ids of rows ts-3 .. (packed documents only)
};

// base + a byte offset held in 32 bits: with a wave-uniform base this is the
// SGPR-base + VGPR-offset addressing form of global memory instructions.
template <typename P>
__device__ __forceinline__ P* at(P* base, uint32_t byte_off) {
  return reinterpret_cast<P*>(reinterpret_cast<typename std::conditional<std::is_const<P>::value, const char, char>::type*>(base) + byte_off);
}

// NPL consecutive floats of LDS (16- or 8-byte aligned).
template <int NPL>
__device__ __forceinline__ void lds_read(const float* p, float (&v)[NPL]) {
  if (NPL == 4) {
    const float4 q = *reinterpret_cast<const float4*>(p);
    v[0] = q.x; v[1] = q.y; v[2] = q.z; v[3] = q.w;
  } else {
    const float2 q = *reinterpret_cast<const float2*>(p);
    v[0] = q.x; v[1] = q.y;
  }
}

// SEQ: packed documents (niverel-mamba 0.1.0 PKG-INFO, "seq_idx strict
// reset"): where the id changes at t, the conv window of t and later steps
// sees zeros before t, and the state is multiplied by 0 before the update of
// t (with one document: multiplied by exactly 1, the same arithmetic).
// XIN: the input is already the activated conv output xc (no conv, no SiLU,
// no conv state written; never with SEQ).
template <int IO, int N, int PASS, bool SEQ, bool XIN = false>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(MSCAN_QUAD_WAVES_PER_EU, MSCAN_QUAD_WAVES_PER_EU))) void scan_quad_kernel(
    int32_t seqlen, int32_t d_inner, int32_t n_chunks, int32_t chunk_len, int32_t bcs,
    const typename Io<IO>::T* __restrict__ x, const typename Io<IO>::T* __restrict__ dt,
    const typename Io<IO>::T* __restrict__ z, const typename Io<IO>::T* __restrict__ Bm,
    const typename Io<IO>::T* __restrict__ Cm, const float* __restrict__ conv_w,
    const float* __restrict__ conv_b, const float* __restrict__ dt_bias,
    const float* __restrict__ Dskip, const float* __restrict__ A,
    const float* conv0,  // conv history before t = 0, [batch][d_inner][3], or NULL = zeros
    const float* h0,     // SSM state before t = 0, [batch][d_inner][N], or NULL = zeros
    typename Io<IO>::T* __restrict__ y, float* conv_state_out, float* ssm_state_out,
    float* __restrict__ sum_S,      // [batch][n_chunks-1][d_inner][N]
    float* __restrict__ sum_delta,  // [batch][n_chunks-1][d_inner]
    float* __restrict__ sum_reset,  // [batch][n_chunks-1][d_inner]: 1 = chunk holds a document start
    const int32_t* __restrict__ seq_idx)  // [batch][seqlen] (SEQ only)
{
  using T = typename Io<IO>::T;
  constexpr int NPL = N / kG;                 // states per lane
  constexpr int kCPB = kThreads / kG;         // channels per workgroup
  constexpr int kTile = kStage * N;           // elements of one staged B or C tile
  constexpr int kEPT = (2 * kTile + kThreads - 1) / kThreads;  // B/C elements per thread
  constexpr int kXE = (kStage + 3) * kCPB;    // x tile elements
  constexpr int kDE = kStage * kCPB;          // dt (and z) tile elements
  constexpr int kNX = (kXE + kThreads - 1) / kThreads;
  constexpr int kND = kDE / kThreads;
  __shared__ Tiles<N> lds;

  const int tid = threadIdx.x;
  const int g = tid & (kG - 1);
  const bool bit0 = (g & 1) != 0, bit1 = (g & 2) != 0;
  const int32_t D = d_inner;
  const int32_t d_raw = blockIdx.x * kCPB + (tid >> 2);
  const bool active = d_raw < D;
  const int32_t d = active ? d_raw : D - 1;  // idle lanes mirror a valid channel and store nothing
  const int32_t chunk = blockIdx.y;
  const int32_t b = blockIdx.z;
  const int32_t t0 = chunk * chunk_len;
  const int32_t t1 = min(t0 + chunk_len, seqlen);
  const size_t bd = static_cast<size_t>(b) * D + d;
  const size_t row0 = static_cast<size_t>(b) * seqlen;

  // per-channel parameters (every lane of the quad needs them for its own timestep)
  const float w0 = XIN ? 0.0f : conv_w[d * 4 + 0], w1 = XIN ? 0.0f : conv_w[d * 4 + 1];
  const float w2 = XIN ? 0.0f : conv_w[d * 4 + 2], w3 = XIN ? 0.0f : conv_w[d * 4 + 3];
  const float cb = XIN ? 0.0f : conv_b[d];
  const float dtb = dt_bias[d];
  const float dsk = (PASS == kFinal) ? Dskip[d] : 0.0f;
  float A2[NPL];
#pragma unroll
  for (int k = 0; k < NPL; ++k) A2[k] = A[d * N + g * NPL + k] * kLog2e;

  // carry-in
  float h[NPL];
#pragma unroll
  for (int k = 0; k < NPL; ++k) h[k] = 0.0f;
  if (PASS == kFinal) {
    if (h0) {
#pragma unroll
      for (int k = 0; k < NPL; ++k) h[k] = h0[bd * N + g * NPL + k];
    }
    for (int32_t j = 0; j < chunk; ++j) {
      const size_t s = (static_cast<size_t>(b) * (n_chunks - 1) + j) * D + d;
      const float sd = sum_delta[s];
      const bool restart = SEQ && sum_reset[s] != 0.0f;  // a document starts in chunk j
#pragma unroll
      for (int k = 0; k < NPL; ++k)
        h[k] = fmaf(exp2_hw(sd * A2[k]), restart ? 0.0f : h[k], sum_S[s * N + g * NPL + k]);
    }
  }

  constexpr uint32_t es = sizeof(T);
  const int32_t d0 = blockIdx.x * kCPB;  // first channel of the workgroup
  const int cl = tid >> 2;               // channel of this lane within the workgroup

  // --- stage tiles: global -> registers (early) -> LDS (end of stage) -----
  // Thread i moves elements i, i + 256, ... of each tile; a row of 64
  // channels is 64 consecutive elements, so the loads are coalesced. Rows at
  // or past t1 read as 0 through the buffer bound (and are never used).
  struct Pre {
    T bc[kEPT];
    T xv[kNX], dv[kND], zv[kND];
    int32_t sq;
  };
  // document ids of rows ts-3 .. ts+15 (rows before 0 take row 0's id: the
  // conv history belongs to the first document); rows past the end read 0
  const auto rSQ = buf_rsrc(SEQ ? seq_idx + row0 : nullptr, SEQ ? static_cast<int64_t>(seqlen) * 4 : 0);
  // Per-thread element offsets inside a stage tile (loop-invariant), in
  // bytes from the tile's first row at channel d0.
  const uint32_t row_bytes = static_cast<uint32_t>(D) * es;
  const uint32_t max_rows = 0x7FFFFFF0u / row_bytes;  // rows a buffer bound can cover
  uint32_t xoff[kNX], doff[kND], bcoff[kEPT];
#pragma unroll
  for (int e = 0; e < kNX; ++e) {
    const int i = tid + e * kThreads;
    xoff[e] = static_cast<uint32_t>(i / kCPB) * row_bytes + static_cast<uint32_t>(i % kCPB) * es;
  }
#pragma unroll
  for (int e = 0; e < kND; ++e) {
    const int i = tid + e * kThreads;
    doff[e] = static_cast<uint32_t>(i / kCPB) * row_bytes + static_cast<uint32_t>(i % kCPB) * es;
  }
#pragma unroll
  for (int e = 0; e < kEPT; ++e) {  // B / C rows are bcs elements apart
    const int r = (tid + e * kThreads) % kTile;
    bcoff[e] = static_cast<uint32_t>((r / N) * bcs + r % N) * es;
  }
  // Buffer bound (bytes) of `rows` rows of D elements past a row start at
  // channel d0: rows at or past the bound read as 0.
  auto rows_bound = [&](int32_t rows) -> int64_t {
    const uint32_t r = min(static_cast<uint32_t>(rows), max_rows);
    return static_cast<int64_t>(r * row_bytes - static_cast<uint32_t>(d0) * es);
  };
  auto tile_load = [&](Pre& pr, int32_t ts) {
    const int64_t lbc = static_cast<int64_t>(t1 - ts) * bcs * es;
    const auto rB = buf_rsrc(Bm + (row0 + ts) * bcs, lbc);
    const auto rC = buf_rsrc(Cm + (row0 + ts) * bcs, lbc);
    // kTile is a multiple of 64, so the tensor of an element is wave-uniform
    static_assert(kTile % 64 == 0, "B/C tile rows must not straddle a wave");
#pragma unroll
    for (int e = 0; e < kEPT; ++e) {
      const int tens = __builtin_amdgcn_readfirstlane((tid + e * kThreads) / kTile);
      pr.bc[e] = buf_load<IO>(tens == 0 ? rB : rC, bcoff[e], 0);
    }
    if (ts >= 3) {  // wave-uniform
      const auto rx = buf_rsrc(x + (row0 + ts - 3) * D + d0, rows_bound(t1 - ts + 3));
#pragma unroll
      for (int e = 0; e < kNX; ++e) pr.xv[e] = buf_load<IO>(rx, xoff[e], 0);
    } else {
      // first stage of the sequence: tile rows before 0 are filled from the
      // conv history when stored; load row 0 in their place
      const int32_t xskip = 3 - ts;
      const auto rx = buf_rsrc(x + row0 * D + d0, rows_bound(t1));
#pragma unroll
      for (int e = 0; e < kNX; ++e) {
        const int i = tid + e * kThreads;
        const int rr = i / kCPB - xskip;
        pr.xv[e] = buf_load<IO>(rx, rr < 0 ? 0u : xoff[e] - static_cast<uint32_t>(xskip) * row_bytes, 0);
      }
    }
    const int64_t lim = rows_bound(t1 - ts);
    const auto rdt = buf_rsrc(dt + (row0 + ts) * D + d0, lim);
    const auto rz = buf_rsrc(z + (row0 + ts) * D + d0, lim);
#pragma unroll
    for (int e = 0; e < kND; ++e) {
      pr.dv[e] = buf_load<IO>(rdt, doff[e], 0);
      if (PASS == kFinal) pr.zv[e] = buf_load<IO>(rz, doff[e], 0);
    }
    if (SEQ && tid < kStage + 3) pr.sq = buf_load_i32(rSQ, static_cast<uint32_t>(max(ts - 3 + tid, 0)) * 4u);
  };
  auto tile_store = [&](const Pre& pr, int buf, int32_t ts) {
#pragma unroll
    for (int e = 0; e < kEPT; ++e) {
      const int i = tid + e * kThreads;
      const int r = i % kTile;
      lds.bc[buf][i / kTile][r / N][r % N] = Io<IO>::cvt(pr.bc[e]);
    }
#pragma unroll
    for (int e = 0; e < kNX; ++e) {
      const int i = tid + e * kThreads;
      if (i < kXE) {
        const int rr = i / kCPB, cc = i % kCPB;
        float v = Io<IO>::cvt(pr.xv[e]);
        const int32_t row = ts - 3 + rr;
        if (row < 0) {  // conv history entry 3 + row of channel d0 + cc
          const int32_t dc = min(d0 + cc, D - 1);
          v = conv0 ? conv0[(static_cast<size_t>(b) * D + dc) * 3 + 3 + row] : 0.0f;
        }
        lds.xt[buf][rr][cc] = v;
      }
    }
#pragma unroll
    for (int e = 0; e < kND; ++e) {
      const int i = tid + e * kThreads;
      lds.dtt[buf][i / kCPB][i % kCPB] = Io<IO>::cvt(pr.dv[e]);
      if (PASS == kFinal) lds.zt[buf][i / kCPB][i % kCPB] = Io<IO>::cvt(pr.zv[e]);
    }
    if (SEQ && tid < kStage + 3) lds.sq[buf][tid] = pr.sq;
  };

  float sd_acc = 0.0f;
  float rs_acc = 0.0f;  // 1 once a document starts in this chunk (summary pass, SEQ)
  // Inputs of this lane's own timestep (ts + 4q + g) in block q.
  struct Own {
    float xw[4], dt, z;
    int32_t s[4];  // document ids of t-3 .. t (SEQ)
  };
  auto own_read = [&](int q, int buf, Own& o) {  // LDS -> registers
#pragma unroll
    for (int k = 0; k < 4; ++k) o.xw[k] = lds.xt[buf][4 * q + g + k][cl];
    o.dt = lds.dtt[buf][4 * q + g][cl];
    o.z = (PASS == kFinal) ? lds.zt[buf][4 * q + g][cl] : 0.0f;
    if (SEQ) {
#pragma unroll
      for (int k = 0; k < 4; ++k) o.s[k] = lds.sq[buf][4 * q + g + k];
    }
  };
  // Per-element terms of the own timestep.
  struct Prep {
    float xc, delta, dx, gz;
    float keep;  // 0 where a document starts (SEQ), else 1
  };
  auto prep = [&](const Own& o) {
    float x0 = o.xw[0], x1 = o.xw[1], x2 = o.xw[2];
    Prep r;
    r.keep = 1.0f;
    if (SEQ) {  // a tap sees x only if no document starts between it and t
      const bool c2 = o.s[2] == o.s[3], c1 = c2 && o.s[1] == o.s[2], c0 = c1 && o.s[0] == o.s[1];
      x2 = c2 ? x2 : 0.0f;
      x1 = c1 ? x1 : 0.0f;
      x0 = c0 ? x0 : 0.0f;
      r.keep = c2 ? 1.0f : 0.0f;
    }
    if (XIN) {
      r.xc = o.xw[3];
    } else {
      float u = fmaf(w0, x0, cb);
      u = fmaf(w1, x1, u);
      u = fmaf(w2, x2, u);
      u = fmaf(w3, o.xw[3], u);
      r.xc = silu(u);
    }
    r.delta = softplus(o.dt + dtb);
    r.dx = r.delta * r.xc;
    r.gz = (PASS == kFinal) ? silu(o.z) : 0.0f;
    return r;
  };
  // B and C of timestep s of the stage, this lane's states.
  struct BC {
    float b[NPL], c[NPL];
  };
  auto bc_read = [&](int st, int buf, BC& v) {
    lds_read<NPL>(&lds.bc[buf][0][st][g * NPL], v.b);
    if (PASS == kFinal) lds_read<NPL>(&lds.bc[buf][1][st][g * NPL], v.c);
  };
  // One timestep (j-th of its block): decay, input, state update and this
  // lane's part of the readout.
  auto step = [&](int j, const Prep& pr, const BC& v, float& pj) {
    float dj = quad_bcast_j(pr.delta, j);
    float dxj = quad_bcast_j(pr.dx, j);
    // Broadcast once into VGPRs (the empty asm keeps the compiler from folding
    // the DPP move into each of the lane's NPL multiplies): on gfx950 an
    // operation with a DPP operand issues at the 16-lane rate, one whose
    // operands are all VGPRs at up to twice that.
    asm("" : "+v"(dj), "+v"(dxj));
    if (SEQ) {  // a document starts at this timestep: state from zero
      const float kj = quad_bcast_j(pr.keep, j);
#pragma unroll
      for (int k = 0; k < NPL; ++k) h[k] *= kj;
    }
#pragma unroll
    for (int k = 0; k < NPL; ++k) {
      const float dA = exp2_hw(dj * A2[k]);
      h[k] = fmaf(dA, h[k], dxj * v.b[k]);
      if (PASS == kFinal) pj = fmaf(v.c[k], h[k], pj);
    }
  };
  // End of a block: the readout sums land in the lane of their timestep,
  // which gates and stores its output (or, in the summary pass, adds its delta).
  auto finish = [&](bool valid, const Prep& pr, const float (&p)[4], __amdgpu_buffer_rsrc_t ry, uint32_t yoff) {
    if (PASS == kSummary) sd_acc += valid ? pr.delta : 0.0f;
    if (PASS == kSummary && SEQ && valid && pr.keep == 0.0f) rs_acc = 1.0f;
    if (PASS == kFinal) {
      const float yv = quad_transpose_sum(p, bit1, bit0);
      const float out = fmaf(dsk, pr.xc, yv) * pr.gz;
      // branch-free: a lane that must not store gets an offset past the range
      buf_store<IO>(out, ry, (active && valid) ? yoff : 0xFFFFFFF0u, 0);
    }
  };

  // y of block q sits 4q + g rows + cl channels past row ts, channel d0
  const uint32_t yoff0 = (static_cast<uint32_t>(g) * static_cast<uint32_t>(D) + static_cast<uint32_t>(cl)) * es;
  const uint32_t yrow4 = 4u * static_cast<uint32_t>(D) * es;

  Pre pre;
  tile_load(pre, t0);
  tile_store(pre, 0, t0);
  __syncthreads();
  int buf = 0;
  for (int32_t ts = t0; ts < t1; ts += kStage) {
    const bool more = ts + kStage < t1;  // wave-uniform
    if (more) tile_load(pre, ts + kStage);
    const auto ry = buf_rsrc(y + (row0 + ts) * D + d0, rows_bound(t1 - ts));
    if (ts + kStage <= t1) {
      // Full stage, software-pipelined: a block's per-element terms are
      // computed during the block before (so its steps start at once) and
      // each timestep's B/C is read one timestep ahead.
      Own own;
      BC bc_c, bc_n;
      own_read(0, buf, own);
      bc_read(0, buf, bc_c);
      Prep pr_c = prep(own);
#pragma unroll
      for (int q = 0; q < kStage / kG; ++q) {
        Prep pr_n = pr_c;
        if (q + 1 < kStage / kG) {
          own_read(q + 1, buf, own);
          pr_n = prep(own);
        }
        float p[4] = {0.0f, 0.0f, 0.0f, 0.0f};
        // Wave priorities (s_setprio): the block's state updates (the
        // dependent chain) first, its readout and the next block's terms
        // second, the tile staging third, the rest last (measured on the
        // long prefill: ~785 -> ~735 us, results bit for bit the same).
        __builtin_amdgcn_s_setprio(3);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int st = 4 * q + j;
          if (st + 1 < kStage) bc_read(st + 1, buf, bc_n);
          __builtin_amdgcn_sched_barrier(0);
          step(j, pr_c, bc_c, p[j]);
          bc_c = bc_n;
        }
        __builtin_amdgcn_s_setprio(2);
        finish(true, pr_c, p, ry, yoff0 + q * yrow4);
        pr_c = pr_n;
      }
    } else {
      // Last (partial) stage of a chunk: timesteps at or past t1 are skipped.
#pragma unroll
      for (int q = 0; q < kStage / kG; ++q) {
        const int32_t tb = ts + 4 * q;
        if (tb < t1) {  // wave-uniform
          Own own;
          own_read(q, buf, own);
          const Prep pr = prep(own);
          float p[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            if (tb + j < t1) {  // wave-uniform
              BC v;
              bc_read(4 * q + j, buf, v);
              step(j, pr, v, p[j]);
            }
          }
          finish(tb + g < t1, pr, p, ry, yoff0 + q * yrow4);
        }
      }
    }
    __builtin_amdgcn_s_setprio(1);
    if (more) tile_store(pre, buf ^ 1, ts + kStage);
    __syncthreads();
    __builtin_amdgcn_s_setprio(0);
    buf ^= 1;
  }

  if (PASS == kSummary) {
    // quad sum of the deltas (each lane holds its own timesteps' share)
    sd_acc += quad_xor1(sd_acc);
    sd_acc += quad_xor2(sd_acc);
    if (SEQ) {
      rs_acc = fmaxf(rs_acc, quad_xor1(rs_acc));
      rs_acc = fmaxf(rs_acc, quad_xor2(rs_acc));
    }
    if (!active) return;
    const size_t s = (static_cast<size_t>(b) * (n_chunks - 1) + chunk) * D + d;
#pragma unroll
    for (int k = 0; k < NPL; ++k) sum_S[s * N + g * NPL + k] = h[k];
    if (g == 0) sum_delta[s] = sd_acc;
    if (SEQ && g == 0) sum_reset[s] = rs_acc;
  } else if (chunk == n_chunks - 1 && active) {
    if (ssm_state_out) {
#pragma unroll
      for (int k = 0; k < NPL; ++k) ssm_state_out[bd * N + g * NPL + k] = h[k];
    }
    if (!XIN && conv_state_out && g < 3) {
      // the last 3 inputs of (history ++ x), copied exactly
      const int32_t r = seqlen - 3 + g;
      float c = 0.0f;
      if (r >= 0) {
        c = Io<IO>::load(x + (row0 + r) * D + d);  // after the loop: plain load
      } else if (conv0) {
        c = conv0[bd * 3 + 3 + r];
      }
      if (SEQ) {  // zero if a document starts after position r
        for (int32_t t = max(r + 1, 1); t < seqlen; ++t)
          if (seq_idx[row0 + t] != seq_idx[row0 + t - 1]) c = 0.0f;
      }
      conv_state_out[bd * 3 + g] = c;
    }
  }
}

template <int IO, int N>
hipError_t launch_typed(const FwdCall& c, const FwdPlan& p) {
  using T = typename Io<IO>::T;
  const unsigned wgs = static_cast<unsigned>((c.d_inner + 63) / 64);
  const T* x = static_cast<const T*>(c.x);
  const T* dt = static_cast<const T*>(c.dt);
  const T* z = static_cast<const T*>(c.z);
  const T* Bm = static_cast<const T*>(c.B);
  const T* Cm = static_cast<const T*>(c.C);
  T* y = static_cast<T*>(c.y);
  const float* conv0 = c.conv_state_in;
  const float* h0 = c.ssm_state_in;
  float* sum_S = nullptr;
  float* sum_delta = nullptr;
  float* sum_reset = nullptr;
  const bool seq = c.seq_idx != nullptr;
  if (p.n_chunks > 1) {
    const QuadWs w = quad_ws_layout(c.batch, c.d_inner, c.d_state, p.n_chunks);
    sum_S = c.workspace + w.sum_S;
    sum_delta = c.workspace + w.sum_delta;
    sum_reset = c.workspace + w.sum_reset;
    // The final pass reads the incoming states in its first chunk while its
    // last chunk may write the outputs in place: give it private copies.
    const size_t bd = static_cast<size_t>(c.batch) * c.d_inner;
    if (c.conv_state_in) {
      hipError_t e = hipMemcpyAsync(c.workspace + w.conv_copy, c.conv_state_in, bd * 3 * sizeof(float),
                                    hipMemcpyDeviceToDevice, c.stream);
      if (e != hipSuccess) return e;
      conv0 = c.workspace + w.conv_copy;
    }
    if (c.ssm_state_in) {
      hipError_t e = hipMemcpyAsync(c.workspace + w.ssm_copy, c.ssm_state_in, bd * N * sizeof(float),
                                    hipMemcpyDeviceToDevice, c.stream);
      if (e != hipSuccess) return e;
      h0 = c.workspace + w.ssm_copy;
    }
    const dim3 grid1(wgs, static_cast<unsigned>(p.n_chunks - 1), static_cast<unsigned>(c.batch));
    auto k1 = c.xc_input ? scan_quad_kernel<IO, N, kSummary, false, true>
              : seq ? scan_quad_kernel<IO, N, kSummary, true> : scan_quad_kernel<IO, N, kSummary, false>;
    hipLaunchKernelGGL(k1, grid1, dim3(kThreads), 0, c.stream, c.seqlen, c.d_inner, p.n_chunks, p.chunk_len, c.bc_stride, x,
                       dt, z, Bm, Cm, c.conv_w, c.conv_b, c.dt_bias, c.D, c.A, conv0, h0, y, c.conv_state_out,
                       c.ssm_state_out, sum_S, sum_delta, sum_reset, c.seq_idx);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  const dim3 grid2(wgs, static_cast<unsigned>(p.n_chunks), static_cast<unsigned>(c.batch));
  auto k2 = c.xc_input ? scan_quad_kernel<IO, N, kFinal, false, true>
            : seq ? scan_quad_kernel<IO, N, kFinal, true> : scan_quad_kernel<IO, N, kFinal, false>;
  hipLaunchKernelGGL(k2, grid2, dim3(kThreads), 0, c.stream, c.seqlen, c.d_inner, p.n_chunks, p.chunk_len, c.bc_stride, x, dt,
                     z, Bm, Cm, c.conv_w, c.conv_b, c.dt_bias, c.D, c.A, conv0, h0, y, c.conv_state_out,
                     c.ssm_state_out, sum_S, sum_delta, sum_reset, c.seq_idx);
  return hipGetLastError();
}

}  // namespace

QuadWs quad_ws_layout(int32_t batch, int32_t d_inner, int32_t d_state, int32_t n_chunks) {
  QuadWs w{};
  if (n_chunks <= 1) return w;
  const size_t bd = static_cast<size_t>(batch) * d_inner;
  const size_t nc1 = static_cast<size_t>(n_chunks - 1);
  w.sum_S = 0;
  w.sum_delta = w.sum_S + bd * nc1 * d_state;
  w.sum_reset = w.sum_delta + bd * nc1;  // 1.0 where a chunk holds a document start
  w.ssm_copy = w.sum_reset + bd * nc1;
  w.conv_copy = w.ssm_copy + bd * d_state;
  w.total = w.conv_copy + bd * 3;
  return w;
}

hipError_t launch_fwd_quad(const FwdCall& c, const FwdPlan& p) {
  if (c.io_dtype == 0) return c.d_state == 16 ? launch_typed<0, 16>(c, p) : launch_typed<0, 8>(c, p);
  return c.d_state == 16 ? launch_typed<1, 16>(c, p) : launch_typed<1, 8>(c, p);
}

}  // namespace mscan
