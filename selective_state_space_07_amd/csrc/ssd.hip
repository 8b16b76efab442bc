// Mamba-2 SSD scan for gfx950 in its chunked form, on the matrix cores.
//
// Per batch row b and head h (scalar A[h]; B and C shared by the heads of a
// group), with S a headdim x d_state state matrix (niverel-mamba 0.1.0
// PKG-INFO, "The weight contract" and "What is *not* promised"):
//   delta_t = softplus(dt_t + dt_bias[h]),  S_t = exp(delta_t A) S_{t-1} + delta_t x_t B_t^T,
//   y_t = S_t C_t + D[h] x_t.
// Over a chunk of Q = 256 steps with cs_t the inclusive cumulative sum of
// delta A inside the chunk, this is exactly (up to rounding)
//   y_t = sum_{s<=t} (C_t . B_s) exp(cs_t - cs_s) delta_s x_s          (intra-chunk)
//       + exp(cs_t) S_in C_t + D x_t                                    (carried state)
//   S_out = exp(cs_end) S_in + sum_s exp(cs_end - cs_s) delta_s x_s B_s^T
// which is three dense contractions per chunk. Three kernels:
//  1. ssd_state_kernel (one workgroup per (b, chunk, head)): the chunk's own
//     end state sum_s exp(cs_end - cs_s) delta_s x_s B_s^T, a [d_state x 64]
//     product with K = Q on MFMA, and the chunk decay exp(cs_end);
//  2. ssd_pass_kernel: the carried state of every chunk, S_in(c+1) =
//     exp(cs_end(c)) S_in(c) + S_local(c), a short sequential pass per (b, h)
//     that overwrites each chunk's local state with its incoming one;
//  3. ssd_out_kernel (one workgroup per (b, chunk, head, 64-step tile)): the
//     carried-state term (C S_in^T on MFMA), then for every 64-step tile s of
//     the chunk up to the own one, G = C_t B_s^T on MFMA, the causal mask,
//     decay exp(cs_t - cs_s) and delta_s applied to G in float32, and G x_s on
//     MFMA; plus D x.
// For bfloat16 io every float32 intermediate that feeds the matrix cores (G,
// the weighted x of kernel 1, the carried state) is split into a bfloat16 hi
// and lo part and multiplied twice, so the products keep ~16 bits of it; the io
// inputs are exact in bfloat16.
// MFMA operands are 8 consecutive k-values per lane (16x16x32 bf16, or eight
// 16x16x4 f32 steps over the same 8 values for float32 io), staged in LDS
// row-major with k contiguous. G is produced transposed (G^T = B_s C_t^T), so
// its accumulators are already the A operand of the next product when the K
// order of that product is permuted to match (slots 0-3: the first 16-row tile,
// slots 4-7: the second); the x operand is read in the same order.
#include "scan_device.h"
#include "scan_internal.h"

namespace mscan {

namespace {

constexpr int kQ = 256;       // chunk length
constexpr int kTile = 64;     // t- and s-tile of the output kernel
constexpr int kP = 64;        // headdim
constexpr int kThreads = 256; // four waves
constexpr int kPad = 8;       // LDS row padding, elements

typedef float f4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf8 __attribute__((ext_vector_type(8)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));
typedef uint32_t u2 __attribute__((ext_vector_type(2)));

// An MFMA operand: 8 k-values of one row (A) or one column (B).
template <int IO>
struct Frag;
template <>
struct Frag<1> {
  bf8 v;
};
template <>
struct Frag<0> {
  f4 lo, hi;
};

__device__ __forceinline__ Frag<1> frag8(const uint16_t* p) {  // 16-byte aligned
  return Frag<1>{__builtin_bit_cast(bf8, *reinterpret_cast<const u4*>(p))};
}
__device__ __forceinline__ Frag<0> frag8(const float* p) {  // 16-byte aligned
  return Frag<0>{*reinterpret_cast<const f4*>(p), *reinterpret_cast<const f4*>(p + 4)};
}
// 4 + 4 values (the permuted K order)
__device__ __forceinline__ Frag<1> frag44(const uint16_t* p0, const uint16_t* p1) {  // 8-byte aligned
  const u2 a = *reinterpret_cast<const u2*>(p0), b = *reinterpret_cast<const u2*>(p1);
  const u4 v = {a.x, a.y, b.x, b.y};
  return Frag<1>{__builtin_bit_cast(bf8, v)};
}
__device__ __forceinline__ Frag<0> frag44(const float* p0, const float* p1) {  // 16-byte aligned
  return Frag<0>{*reinterpret_cast<const f4*>(p0), *reinterpret_cast<const f4*>(p1)};
}
// from registers (float), rounded to the operand type
template <int IO>
__device__ __forceinline__ Frag<IO> frag_regs(f4 lo, f4 hi);
template <>
__device__ __forceinline__ Frag<1> frag_regs<1>(f4 lo, f4 hi) {
  bf8 v;
  v[0] = static_cast<__bf16>(lo.x);
  v[1] = static_cast<__bf16>(lo.y);
  v[2] = static_cast<__bf16>(lo.z);
  v[3] = static_cast<__bf16>(lo.w);
  v[4] = static_cast<__bf16>(hi.x);
  v[5] = static_cast<__bf16>(hi.y);
  v[6] = static_cast<__bf16>(hi.z);
  v[7] = static_cast<__bf16>(hi.w);
  return Frag<1>{v};
}
template <>
__device__ __forceinline__ Frag<0> frag_regs<0>(f4 lo, f4 hi) {
  return Frag<0>{lo, hi};
}
// A float32 operand as the sum of two bfloat16 operands (hi = RNE(v), lo =
// RNE(v - hi)): two products on the bfloat16 matrix cores then carry about 16
// significant bits of v instead of 8. Used wherever an operand is a float32
// intermediate (the decayed G, the weighted x, the carried state); the io
// inputs themselves are exact in bfloat16.
struct Split {
  Frag<1> hi, lo;
};
__device__ __forceinline__ float bf_round(float v) { return static_cast<float>(static_cast<__bf16>(v)); }
__device__ __forceinline__ Split split8(f4 a, f4 b) {
  const f4 ah = {bf_round(a.x), bf_round(a.y), bf_round(a.z), bf_round(a.w)};
  const f4 bh = {bf_round(b.x), bf_round(b.y), bf_round(b.z), bf_round(b.w)};
  return Split{frag_regs<1>(ah, bh), frag_regs<1>(a - ah, b - bh)};
}
__device__ __forceinline__ f4 mma(const Frag<1>& a, const Frag<1>& b, f4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, b.v, c, 0, 0, 0);
}
__device__ __forceinline__ f4 mma(const Frag<0>& a, const Frag<0>& b, f4 c) {
  // slot j of every lane group feeds step j: the eight steps cover all 32 k
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo.x, b.lo.x, c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo.y, b.lo.y, c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo.z, b.lo.z, c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo.w, b.lo.w, c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi.x, b.hi.x, c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi.y, b.hi.y, c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi.z, b.hi.z, c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi.w, b.hi.w, c, 0, 0, 0);
  return c;
}

// acc += A B where A is a float32 operand given in registers (8 values of the
// lane's row) and B an io operand; for bfloat16 io A is split into hi + lo.
template <int IO>
__device__ __forceinline__ f4 mma_f32a(f4 a_lo4, f4 a_hi4, const Frag<IO>& b, f4 c);
template <>
__device__ __forceinline__ f4 mma_f32a<1>(f4 a_lo4, f4 a_hi4, const Frag<1>& b, f4 c) {
  const Split a = split8(a_lo4, a_hi4);
  return mma(a.lo, b, mma(a.hi, b, c));
}
template <>
__device__ __forceinline__ f4 mma_f32a<0>(f4 a_lo4, f4 a_hi4, const Frag<0>& b, f4 c) {
  return mma(Frag<0>{a_lo4, a_hi4}, b, c);
}
// acc += A B where A is an io operand and B a float32 operand (8 values of the
// lane's column) read from 16-byte aligned memory.
template <int IO>
__device__ __forceinline__ f4 mma_f32b(const Frag<IO>& a, const float* p, f4 c);
template <>
__device__ __forceinline__ f4 mma_f32b<1>(const Frag<1>& a, const float* p, f4 c) {
  const Split b = split8(*reinterpret_cast<const f4*>(p), *reinterpret_cast<const f4*>(p + 4));
  return mma(a, b.lo, mma(a, b.hi, c));
}
template <>
__device__ __forceinline__ f4 mma_f32b<0>(const Frag<0>& a, const float* p, f4 c) {
  return mma(a, frag8(p), c);
}

// Inclusive prefix sum over the workgroup's 256 threads (one value each), in a
// fixed order: within each wave by shuffles, then the wave totals.
__device__ __forceinline__ float block_scan(float v, float* wsum, int tid) {
  const int lane = tid & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const float u = __shfl_up(v, o, 64);
    if (lane >= o) v += u;
  }
  if (lane == 63) wsum[tid >> 6] = v;
  __syncthreads();
  float off = 0.0f;
  for (int w = 0; w < (tid >> 6); ++w) off += wsum[w];
  return v + off;
}

// delta and the cumulative log-decay cs of one chunk into LDS (thread = step).
template <int IO>
__device__ __forceinline__ void chunk_decay(float* cs, float* dl, float* wsum, const typename Io<IO>::T* dt,
                                            int64_t dt_index, int32_t nheads, int valid, float bias, float A,
                                            int tid) {
  float delta = 0.0f;
  if (tid < valid) delta = softplus(Io<IO>::load(dt + dt_index + static_cast<int64_t>(tid) * nheads) + bias);
  const float c = block_scan(delta * A, wsum, tid);
  cs[tid] = c;
  dl[tid] = delta;
  __syncthreads();
}

// Rows 0..63 of a row-major io matrix (row stride `ld` elements, W columns)
// into LDS rows of W + kPad; rows at or past `rows` are zero.
template <int IO, int W>
__device__ __forceinline__ void stage_rows(typename Io<IO>::T* lds, const typename Io<IO>::T* g, int64_t ld, int rows,
                                           int tid) {
  using T = typename Io<IO>::T;
  constexpr int kVec = 16 / static_cast<int>(sizeof(T));
  constexpr int kPer = W / kVec;
  for (int i = tid; i < kTile * kPer; i += kThreads) {
    const int r = i / kPer, cc = i - r * kPer;
    u4 v = {0u, 0u, 0u, 0u};
    if (r < rows) v = *reinterpret_cast<const u4*>(g + r * ld + cc * kVec);
    *reinterpret_cast<u4*>(lds + r * (W + kPad) + cc * kVec) = v;
  }
}

// Transpose rows 0..63 (W columns) of a row-major io matrix into LDS as
// [W][kTile + kPad], each row s scaled by scale[s]; rows past `rows` are zero.
template <int IO, int W>
__device__ __forceinline__ void stage_cols(typename Io<IO>::T* lds, const typename Io<IO>::T* g, int64_t ld, int rows,
                                           const float* scale, int tid) {
  using T = typename Io<IO>::T;
  constexpr int kVec = 16 / static_cast<int>(sizeof(T));
  constexpr int kPer = W / kVec;
  for (int i = tid; i < kTile * kPer; i += kThreads) {
    const int r = i / kPer, c0 = (i - r * kPer) * kVec;
    u4 v = {0u, 0u, 0u, 0u};
    if (r < rows) v = *reinterpret_cast<const u4*>(g + r * ld + c0);
    const float w = scale ? scale[r] : 1.0f;
    const T* e = reinterpret_cast<const T*>(&v);
#pragma unroll
    for (int j = 0; j < kVec; ++j) {
      if constexpr (IO == 0) {
        lds[(c0 + j) * (kTile + kPad) + r] = w * e[j];
      } else {
        lds[(c0 + j) * (kTile + kPad) + r] = scale ? Io<1>::from_float(w * Io<1>::cvt(e[j])) : e[j];
      }
    }
  }
}

// Transpose rows 0..63 (W columns) of a row-major io matrix into float32 LDS
// as [W][kTile + kPad], each row s scaled by scale[s]; rows past `rows` are zero.
template <int IO, int W>
__device__ __forceinline__ void stage_cols_f32(float* lds, const typename Io<IO>::T* g, int64_t ld, int rows,
                                               const float* scale, int tid) {
  using T = typename Io<IO>::T;
  constexpr int kVec = 16 / static_cast<int>(sizeof(T));
  constexpr int kPer = W / kVec;
  for (int i = tid; i < kTile * kPer; i += kThreads) {
    const int r = i / kPer, c0 = (i - r * kPer) * kVec;
    u4 v = {0u, 0u, 0u, 0u};
    if (r < rows) v = *reinterpret_cast<const u4*>(g + r * ld + c0);
    const float w = scale[r];
    const T* e = reinterpret_cast<const T*>(&v);
#pragma unroll
    for (int j = 0; j < kVec; ++j) lds[(c0 + j) * (kTile + kPad) + r] = w * Io<IO>::cvt(e[j]);
  }
}

// 1. Local end state of each chunk and its decay.
template <int IO, int N>
__global__ __launch_bounds__(kThreads) void ssd_state_kernel(
    int32_t seqlen, int32_t nheads, int32_t ngroups, int32_t nchunks, const typename Io<IO>::T* __restrict__ x,
    const typename Io<IO>::T* __restrict__ dt, const typename Io<IO>::T* __restrict__ Bm,
    const float* __restrict__ dt_bias, const float* __restrict__ A, float* __restrict__ states,
    float* __restrict__ decay) {
  using T = typename Io<IO>::T;
  constexpr int kNT = N / 64;  // 16-row n-tiles per wave
  __shared__ float cs[kQ], dl[kQ], wgt[kQ], wsum[4];
  __shared__ __align__(16) T bT[N][kTile + kPad];       // B^T of the s-tile: [n][s]
  __shared__ __align__(16) float wT[kP][kTile + kPad];  // (weight x)^T of the s-tile, float32: [p][s]
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, g16 = lane >> 4, c16 = lane & 15;
  const int32_t c = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int32_t grp = h / (nheads / ngroups);
  const int64_t t0 = static_cast<int64_t>(c) * kQ;
  const int valid = static_cast<int>(min(static_cast<int64_t>(kQ), seqlen - t0));
  const int64_t row0 = static_cast<int64_t>(b) * seqlen + t0;
  chunk_decay<IO>(cs, dl, wsum, dt, row0 * nheads + h, nheads, valid, dt_bias[h], A[h], tid);
  const float cs_end = cs[kQ - 1];
  wgt[tid] = exp2_hw((cs_end - cs[tid]) * kLog2e) * dl[tid];
  f4 acc[kNT][4];
#pragma unroll
  for (int nt = 0; nt < kNT; ++nt)
#pragma unroll
    for (int pt = 0; pt < 4; ++pt) acc[nt][pt] = f4{0.0f, 0.0f, 0.0f, 0.0f};
  for (int s0 = 0; s0 < valid; s0 += kTile) {
    __syncthreads();  // previous tile's operands read; wgt written
    const int rows = min(kTile, valid - s0);
    stage_cols<IO, N>(&bT[0][0], Bm + ((row0 + s0) * ngroups + grp) * N, static_cast<int64_t>(ngroups) * N, rows,
                      nullptr, tid);
    stage_cols_f32<IO, kP>(&wT[0][0], x + ((row0 + s0) * nheads + h) * kP, static_cast<int64_t>(nheads) * kP, rows,
                           &wgt[s0], tid);
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < kTile; ks += 32) {
      Frag<IO> a[kNT];
#pragma unroll
      for (int nt = 0; nt < kNT; ++nt) a[nt] = frag8(&bT[(wv * kNT + nt) * 16 + c16][ks + g16 * 8]);
#pragma unroll
      for (int pt = 0; pt < 4; ++pt) {
        const float* bq = &wT[pt * 16 + c16][ks + g16 * 8];
#pragma unroll
        for (int nt = 0; nt < kNT; ++nt) acc[nt][pt] = mma_f32b<IO>(a[nt], bq, acc[nt][pt]);
      }
    }
  }
  // lane holds S[n = tile*16 + 4 g16 + j][p = pt*16 + c16]: four consecutive n of the [p][n] layout
  float* out = states + ((static_cast<int64_t>(b) * nchunks + c) * nheads + h) * kP * N;
#pragma unroll
  for (int nt = 0; nt < kNT; ++nt)
#pragma unroll
    for (int pt = 0; pt < 4; ++pt)
      *reinterpret_cast<f4*>(out + (pt * 16 + c16) * N + (wv * kNT + nt) * 16 + g16 * 4) = acc[nt][pt];
  if (tid == 0) decay[(static_cast<int64_t>(b) * nchunks + c) * nheads + h] = exp2_hw(cs_end * kLog2e);
}

// 2. Carried states: each chunk's local state is replaced by the state that
// enters it; the last one out is the final state.
__global__ __launch_bounds__(kThreads) void ssd_pass_kernel(int32_t nchunks, int32_t nheads, int32_t pn4,
                                                            const float* state_in, float* states,
                                                            const float* __restrict__ decay, float* state_out) {
  const int32_t e = static_cast<int32_t>(blockIdx.x) * kThreads + static_cast<int32_t>(threadIdx.x);
  if (e >= pn4) return;
  const int32_t h = blockIdx.y, b = blockIdx.z;
  const int64_t bh = static_cast<int64_t>(b) * nheads + h;
  f4 H = state_in ? reinterpret_cast<const f4*>(state_in)[bh * pn4 + e] : f4{0.0f, 0.0f, 0.0f, 0.0f};
  for (int32_t c = 0; c < nchunks; ++c) {
    const int64_t bch = (static_cast<int64_t>(b) * nchunks + c) * nheads + h;
    f4* slot = reinterpret_cast<f4*>(states) + bch * pn4 + e;
    const f4 S = *slot;
    *slot = H;
    H = decay[bch] * H + S;
  }
  if (state_out) reinterpret_cast<f4*>(state_out)[bh * pn4 + e] = H;
}

// 3. Outputs of one 64-step tile of a chunk.
template <int IO, int N>
__global__ __launch_bounds__(kThreads) void ssd_out_kernel(
    int32_t seqlen, int32_t nheads, int32_t ngroups, int32_t nchunks, const typename Io<IO>::T* __restrict__ x,
    const typename Io<IO>::T* __restrict__ dt, const typename Io<IO>::T* __restrict__ Bm,
    const typename Io<IO>::T* __restrict__ Cm, const float* __restrict__ dt_bias, const float* __restrict__ A,
    const float* __restrict__ Dskip, const float* __restrict__ states, typename Io<IO>::T* __restrict__ y) {
  using T = typename Io<IO>::T;
  __shared__ float cs[kQ], dl[kQ], wsum[4];
  __shared__ __align__(16) T cT[kTile][N + kPad];   // C rows of the t-tile: [t][n]
  __shared__ __align__(16) T bS[kTile][N + kPad];   // B rows of the s-tile: [s][n]
  __shared__ __align__(16) T xT[kP][kTile + kPad];  // x^T of the s-tile: [p][s]
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, g16 = lane >> 4, c16 = lane & 15;
  const int32_t c = static_cast<int32_t>(blockIdx.x) >> 2, tt = static_cast<int32_t>(blockIdx.x) & 3;
  const int32_t h = blockIdx.y, b = blockIdx.z;
  const int32_t grp = h / (nheads / ngroups);
  const int64_t t0 = static_cast<int64_t>(c) * kQ;
  const int valid = static_cast<int>(min(static_cast<int64_t>(kQ), seqlen - t0));
  if (tt * kTile >= valid) return;  // the whole workgroup, before any barrier
  const int64_t row0 = static_cast<int64_t>(b) * seqlen + t0;
  chunk_decay<IO>(cs, dl, wsum, dt, row0 * nheads + h, nheads, valid, dt_bias[h], A[h], tid);
  const int tb = tt * kTile;  // first step of the t-tile in the chunk
  stage_rows<IO, N>(&cT[0][0], Cm + ((row0 + tb) * ngroups + grp) * N, static_cast<int64_t>(ngroups) * N,
                    min(kTile, valid - tb), tid);
  __syncthreads();

  // carried state: Y[t][p] = exp(cs_t) sum_n C[t][n] S_in[p][n]
  f4 acc[4];
  {
    const float* Sin = states + ((static_cast<int64_t>(b) * nchunks + c) * nheads + h) * kP * N;
#pragma unroll
    for (int pt = 0; pt < 4; ++pt) acc[pt] = f4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int ks = 0; ks < N; ks += 32) {
      const Frag<IO> a = frag8(&cT[wv * 16 + c16][ks + g16 * 8]);
#pragma unroll
      for (int pt = 0; pt < 4; ++pt) acc[pt] = mma_f32b<IO>(a, Sin + (pt * 16 + c16) * N + ks + g16 * 8, acc[pt]);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float e = exp2_hw(cs[tb + wv * 16 + g16 * 4 + j] * kLog2e);
#pragma unroll
      for (int pt = 0; pt < 4; ++pt) acc[pt][j] *= e;
    }
  }

  // intra-chunk: s-tiles up to the own one
  const int tpos = tb + wv * 16 + c16;  // this lane's step as the column of G^T / row of G
  const float cst = cs[tpos];
  for (int sb = 0; sb <= tb; sb += kTile) {
    __syncthreads();  // previous s-tile's operands read
    const int rows = min(kTile, valid - sb);
    stage_rows<IO, N>(&bS[0][0], Bm + ((row0 + sb) * ngroups + grp) * N, static_cast<int64_t>(ngroups) * N, rows, tid);
    stage_cols<IO, kP>(&xT[0][0], x + ((row0 + sb) * nheads + h) * kP, static_cast<int64_t>(nheads) * kP, rows,
                       nullptr, tid);
    __syncthreads();
    // G^T[s][t] = sum_n B[s][n] C[t][n]: lane holds s = si*16 + 4 g16 + j, t = tpos
    f4 gt[4];
#pragma unroll
    for (int si = 0; si < 4; ++si) {
      gt[si] = f4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int ks = 0; ks < N; ks += 32)
        gt[si] = mma(frag8(&bS[si * 16 + c16][ks + g16 * 8]), frag8(&cT[wv * 16 + c16][ks + g16 * 8]), gt[si]);
    }
    // causal mask, decay exp(cs_t - cs_s) and delta_s, in float32
#pragma unroll
    for (int si = 0; si < 4; ++si)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int spos = sb + si * 16 + g16 * 4 + j;
        gt[si][j] = spos <= tpos ? gt[si][j] * (exp2_hw((cst - cs[spos]) * kLog2e) * dl[spos]) : 0.0f;
      }
    // Y[t][p] += sum_s G[t][s] x[s][p], K order: slots 0-3 from tile 2m, 4-7 from tile 2m+1
#pragma unroll
    for (int m = 0; m < 2; ++m) {
#pragma unroll
      for (int pt = 0; pt < 4; ++pt) {
        const T* row = &xT[pt * 16 + c16][0];
        acc[pt] = mma_f32a<IO>(gt[2 * m], gt[2 * m + 1], frag44(row + 32 * m + 4 * g16, row + 32 * m + 16 + 4 * g16),
                               acc[pt]);
      }
    }
  }

  // D skip and store: lane holds Y[t = tb + wv*16 + 4 g16 + j][p = pt*16 + c16]
  const float dsk = Dskip[h];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int tl = tb + wv * 16 + g16 * 4 + j;
    if (tl < valid) {
      const int64_t base = ((row0 + tl) * nheads + h) * kP;
#pragma unroll
      for (int pt = 0; pt < 4; ++pt) {
        const int64_t i = base + pt * 16 + c16;
        Io<IO>::store(y + i, fmaf(dsk, Io<IO>::load(x + i), acc[pt][j]));
      }
    }
  }
}

template <int IO, int N>
hipError_t launch_typed(const SsdCall& c) {
  using T = typename Io<IO>::T;
  const int32_t nchunks = (c.seqlen + kQ - 1) / kQ;
  const SsdWs w = ssd_ws_layout(c.batch, c.seqlen, c.nheads, c.d_state);
  float* states = c.workspace + w.states;
  float* decay = c.workspace + w.decay;
  hipLaunchKernelGGL((ssd_state_kernel<IO, N>), dim3(nchunks, c.nheads, c.batch), dim3(kThreads), 0, c.stream,
                     c.seqlen, c.nheads, c.ngroups, nchunks, static_cast<const T*>(c.x), static_cast<const T*>(c.dt),
                     static_cast<const T*>(c.B), c.dt_bias, c.A, states, decay);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int32_t pn4 = kP * N / 4;
  hipLaunchKernelGGL(ssd_pass_kernel, dim3((pn4 + kThreads - 1) / kThreads, c.nheads, c.batch), dim3(kThreads), 0,
                     c.stream, nchunks, c.nheads, pn4, c.state_in, states, decay, c.state_out);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((ssd_out_kernel<IO, N>), dim3(nchunks * 4, c.nheads, c.batch), dim3(kThreads), 0, c.stream,
                     c.seqlen, c.nheads, c.ngroups, nchunks, static_cast<const T*>(c.x), static_cast<const T*>(c.dt),
                     static_cast<const T*>(c.B), static_cast<const T*>(c.C), c.dt_bias, c.A, c.D, states,
                     static_cast<T*>(c.y));
  return hipGetLastError();
}

}  // namespace

SsdWs ssd_ws_layout(int32_t batch, int32_t seqlen, int32_t nheads, int32_t d_state) {
  SsdWs w{};
  const size_t nchunks = (static_cast<size_t>(seqlen) + kQ - 1) / kQ;
  const size_t bch = static_cast<size_t>(batch) * nchunks * nheads;
  w.states = 0;
  w.decay = bch * kP * d_state;
  w.total = w.decay + ((bch + 63) / 64) * 64;
  return w;
}

hipError_t launch_ssd(const SsdCall& c) {
  if (c.io_dtype == 0) return c.d_state == 64 ? launch_typed<0, 64>(c) : launch_typed<0, 128>(c);
  return c.d_state == 64 ? launch_typed<1, 64>(c) : launch_typed<1, 128>(c);
}

}  // namespace mscan
