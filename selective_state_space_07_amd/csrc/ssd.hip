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
//  3. ssd_out_kernel (one workgroup per (b, chunk, 64-step tile) and one or
//     two heads of a group; each lane keeps its C fragments in registers): the
//     carried-state term (C S_in^T on MFMA), then for every 64-step tile s of
//     the chunk up to the own one, G = C_t B_s^T on MFMA (once for the heads
//     of the workgroup), the causal mask, decay exp(cs_t - cs_s) and delta_s
//     of each head applied to G in float32, and G x_s on MFMA; plus D x.
//     The carried state comes through LDS in double-buffered slices (one
//     barrier per slice), and workgroup ids are ordered so that the four
//     t-tiles of a (b, chunk, head pair), which read the same state and x
//     tiles, run on one XCD and share its L2.
// For bfloat16 io every float32 intermediate that feeds the matrix cores (G,
// the weighted x of kernel 1, the carried state) is split into a bfloat16 hi
// and lo part and multiplied twice, so the products keep ~16 bits of it; the io
// inputs are exact in bfloat16. Each split is made once, where the value is
// produced: by the pass kernel for the carried state, by kernel 1's staging
// for the weighted x, by each lane for its own G accumulators.
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
// Row pitch of the transposed [p][s] tiles that feed the matrix cores: 68
// elements puts the 16 rows one wave reads at once on distinct banks (a pitch
// of 72 would make rows c and c + 8 collide).
constexpr int kPitchT = kTile + 4;

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
template <int IO>
__device__ __forceinline__ Frag<IO> frag_zero();
template <>
__device__ __forceinline__ Frag<1> frag_zero<1>() {
  const u4 z = {0u, 0u, 0u, 0u};
  return Frag<1>{__builtin_bit_cast(bf8, z)};
}
template <>
__device__ __forceinline__ Frag<0> frag_zero<0>() {
  return Frag<0>{f4{0.0f, 0.0f, 0.0f, 0.0f}, f4{0.0f, 0.0f, 0.0f, 0.0f}};
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
// acc += A B where B is a float32 operand (8 values of the lane's column) stored
// pre-split, as the pass kernel stores the carried state and the state kernel
// the weighted x: for bfloat16 io the 8 hi then the 8 lo bfloat16 parts in the
// bytes of 8 floats; for float32 io the 8 floats themselves. 16-byte aligned.
template <int IO>
__device__ __forceinline__ f4 mma_state(const Frag<IO>& a, const float* p, f4 c);
template <>
__device__ __forceinline__ f4 mma_state<1>(const Frag<1>& a, const float* p, f4 c) {
  const uint16_t* q = reinterpret_cast<const uint16_t*>(p);
  return mma(a, frag8(q + 8), mma(a, frag8(q), c));
}
template <>
__device__ __forceinline__ f4 mma_state<0>(const Frag<0>& a, const float* p, f4 c) {
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

// Inclusive running maximum over the workgroup's 256 threads (one value each).
__device__ __forceinline__ float block_scan_max(float v, float* wmax, int tid) {
  const int lane = tid & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const float u = __shfl_up(v, o, 64);
    if (lane >= o) v = fmaxf(v, u);
  }
  if (lane == 63) wmax[tid >> 6] = v;
  __syncthreads();
  for (int w = 0; w < (tid >> 6); ++w) v = fmaxf(v, wmax[w]);
  return v;
}

// Tile staging, split into a global load into registers (issued early, so it
// stays in flight while the previous tile is multiplied) and a store into LDS.
// Loads are branch-free: rows past `rows` read row 0 and are zeroed at store.
// Rows 0..63 of a row-major io matrix (row stride ld, W columns) -> LDS rows
// [64][W + kPad]; consecutive lanes store consecutive 16-byte chunks.
template <int IO, int W>
struct RowTile {
  using T = typename Io<IO>::T;
  static constexpr int kVec = 16 / static_cast<int>(sizeof(T));
  static constexpr int kPer = W / kVec;
  static constexpr int kN = kTile * kPer / kThreads;
  u4 v[kN];
  int rows;
  __device__ __forceinline__ void load(const T* g, int64_t ld, int rows_, int tid) {
    rows = rows_;
#pragma unroll
    for (int q = 0; q < kN; ++q) {
      const int i = tid + q * kThreads, r = i / kPer, cc = i - r * kPer;
      v[q] = *reinterpret_cast<const u4*>(g + (r < rows ? r : 0) * ld + cc * kVec);
    }
  }
  __device__ __forceinline__ void store(T* lds, int tid) const {
#pragma unroll
    for (int q = 0; q < kN; ++q) {
      const int i = tid + q * kThreads, r = i / kPer, cc = i - r * kPer;
      const u4 z = {0u, 0u, 0u, 0u};
      *reinterpret_cast<u4*>(lds + r * (W + kPad) + cc * kVec) = r < rows ? v[q] : z;
    }
  }
};

// Rows 0..63 (W columns) -> LDS transposed, [W][P] io. bfloat16: a
// thread takes rows 2rp and 2rp+1 of one 8-column chunk and stores eight
// 32-bit words (the two rows' values of a column); lanes 0-31 take
// consecutive rp, so a wave's 64 stores hit 64 distinct banks. float32: a
// thread takes one row of a 4-column chunk; lanes take consecutive rows.
template <int IO, int W, int P = kTile + kPad>
struct ColTile;
template <int W, int P>
struct ColTile<1, W, P> {
  static constexpr int kPer = W / 8;
  static constexpr int kN = 32 * kPer / kThreads;
  u4 lo[kN], hi[kN];
  int rows;
  __device__ __forceinline__ void load(const uint16_t* g, int64_t ld, int rows_, int tid) {
    rows = rows_;
#pragma unroll
    for (int q = 0; q < kN; ++q) {
      const int i = tid + q * kThreads, rp = i & 31, cc = i >> 5;
      const int r0 = 2 * rp < rows ? 2 * rp : 0, r1 = 2 * rp + 1 < rows ? 2 * rp + 1 : 0;
      lo[q] = *reinterpret_cast<const u4*>(g + r0 * ld + cc * 8);
      hi[q] = *reinterpret_cast<const u4*>(g + r1 * ld + cc * 8);
    }
  }
  __device__ __forceinline__ void store(uint16_t* lds, int tid) const {
    uint32_t* w = reinterpret_cast<uint32_t*>(lds);
    static_assert(P % 2 == 0, "pairs of bfloat16 per word");
    constexpr int kStrideW = P / 2;
#pragma unroll
    for (int q = 0; q < kN; ++q) {
      const int i = tid + q * kThreads, rp = i & 31, cc = i >> 5;
      const uint32_t m0 = 2 * rp < rows ? 0xFFFFFFFFu : 0u, m1 = 2 * rp + 1 < rows ? 0xFFFFFFFFu : 0u;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint32_t a = lo[q][k] & m0, b = hi[q][k] & m1;
        w[(cc * 8 + 2 * k) * kStrideW + rp] = (a & 0xFFFFu) | (b << 16);
        w[(cc * 8 + 2 * k + 1) * kStrideW + rp] = (a >> 16) | (b & 0xFFFF0000u);
      }
    }
  }
};
template <int W, int P>
struct ColTile<0, W, P> {
  static constexpr int kPer = W / 4;
  static constexpr int kN = kTile * kPer / kThreads;
  u4 v[kN];
  int rows;
  __device__ __forceinline__ void load(const float* g, int64_t ld, int rows_, int tid) {
    rows = rows_;
#pragma unroll
    for (int q = 0; q < kN; ++q) {
      const int i = tid + q * kThreads, r = i & 63, cc = i >> 6;
      v[q] = *reinterpret_cast<const u4*>(g + (r < rows ? r : 0) * ld + cc * 4);
    }
  }
  __device__ __forceinline__ void store(float* lds, int tid) const {
#pragma unroll
    for (int q = 0; q < kN; ++q) {
      const int i = tid + q * kThreads, r = i & 63, cc = i >> 6;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        // element copied out first: a bit_cast applied to the vector element
        // itself read element 0 for every k
        const uint32_t e = v[q][k];
        lds[(cc * 4 + k) * P + r] = r < rows ? __builtin_bit_cast(float, e) : 0.0f;
      }
    }
  }
};

// Rows 0..63 (64 columns) of an io matrix -> float32 LDS transposed,
// [64][kPitchT], row s scaled by scale[s]; lanes take consecutive rows.
template <int IO>
struct WeightedColTile {
  using T = typename Io<IO>::T;
  static constexpr int kVec = 16 / static_cast<int>(sizeof(T));
  static constexpr int kPer = kP / kVec;
  static constexpr int kN = kTile * kPer / kThreads;
  u4 v[kN];
  int rows;
  __device__ __forceinline__ void load(const T* g, int64_t ld, int rows_, int tid) {
    rows = rows_;
#pragma unroll
    for (int q = 0; q < kN; ++q) {
      const int i = tid + q * kThreads, r = i & 63, cc = i >> 6;
      v[q] = *reinterpret_cast<const u4*>(g + (r < rows ? r : 0) * ld + cc * kVec);
    }
  }
  __device__ __forceinline__ void store(float* lds, const float* scale, int tid) const {
#pragma unroll
    for (int q = 0; q < kN; ++q) {
      const int i = tid + q * kThreads, r = i & 63, cc = i >> 6;
      const float w = r < rows ? scale[r] : 0.0f;
      const T* e = reinterpret_cast<const T*>(&v[q]);
#pragma unroll
      for (int k = 0; k < kVec; ++k) lds[(cc * kVec + k) * kPitchT + r] = w * Io<IO>::cvt(e[k]);
    }
  }
};

// bfloat16 io: rows 0..63 (64 columns p) of x, row s scaled by scale[s], ->
// LDS transposed and already split into matrix-core operand parts: row p
// (kPitchT words), 8-step group g at word 8g: words 0-3 the hi parts of
// steps 8g .. 8g+7 (two per word), words 4-7 the lo parts. A thread takes
// steps 2rp and 2rp+1 of one 8-column chunk, so it packs each pair itself.
struct WeightedSplitTile {
  u4 v0, v1;  // rows 2rp and 2rp+1, columns 8cc .. 8cc+7
  int rows;
  __device__ __forceinline__ void load(const uint16_t* g, int64_t ld, int rows_, int tid) {
    rows = rows_;
    const int rp = tid & 31, cc = tid >> 5;
    const int r0 = 2 * rp < rows ? 2 * rp : 0, r1 = 2 * rp + 1 < rows ? 2 * rp + 1 : 0;
    v0 = *reinterpret_cast<const u4*>(g + r0 * ld + cc * 8);
    v1 = *reinterpret_cast<const u4*>(g + r1 * ld + cc * 8);
  }
  __device__ __forceinline__ void store(float* lds, const float* scale, int tid) const {
    static_assert(32 * 8 == kThreads, "one 2 x 8 block per thread");
    uint32_t* w = reinterpret_cast<uint32_t*>(lds);
    const int rp = tid & 31, cc = tid >> 5;
    const float w0 = 2 * rp < rows ? scale[2 * rp] : 0.0f, w1 = 2 * rp + 1 < rows ? scale[2 * rp + 1] : 0.0f;
    const uint16_t* e0 = reinterpret_cast<const uint16_t*>(&v0);
    const uint16_t* e1 = reinterpret_cast<const uint16_t*>(&v1);
    const int off = (rp >> 2) * 8 + (rp & 3);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const float a = w0 * Io<1>::cvt(e0[k]), b = w1 * Io<1>::cvt(e1[k]);
      const __bf16 ah = static_cast<__bf16>(a), bh = static_cast<__bf16>(b);
      const __bf16 al = static_cast<__bf16>(a - static_cast<float>(ah));
      const __bf16 bl = static_cast<__bf16>(b - static_cast<float>(bh));
      const uint32_t hi = static_cast<uint32_t>(__builtin_bit_cast(uint16_t, ah)) |
                          (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, bh)) << 16);
      const uint32_t lo = static_cast<uint32_t>(__builtin_bit_cast(uint16_t, al)) |
                          (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, bl)) << 16);
      uint32_t* row = w + (cc * 8 + k) * kPitchT;
      row[off] = hi;
      row[off + 4] = lo;
    }
  }
};
// The state kernel's weighted-x tile: pre-split for bfloat16 io, float32 otherwise.
template <int IO>
struct WeightedTile;
template <>
struct WeightedTile<1> {
  using type = WeightedSplitTile;
};
template <>
struct WeightedTile<0> {
  using type = WeightedColTile<0>;
};

// Columns k0 .. k0+W-1 of the float32 carried state S_in [64][N] -> LDS
// [64][W + 4]; W/4 consecutive lanes store one row (16 bytes each).
template <int W>
struct StateSlice {
  static constexpr int kPerRow = W / 4;
  static constexpr int kN = kP * kPerRow / kThreads;
  u4 v[kN];
  __device__ __forceinline__ void load(const float* g, int n, int k0, int tid) {
#pragma unroll
    for (int q = 0; q < kN; ++q) {
      const int i = tid + q * kThreads, r = i / kPerRow, cc = i - r * kPerRow;
      v[q] = *reinterpret_cast<const u4*>(g + r * n + k0 + cc * 4);
    }
  }
  __device__ __forceinline__ void store(float* lds, int tid) const {
#pragma unroll
    for (int q = 0; q < kN; ++q) {
      const int i = tid + q * kThreads, r = i / kPerRow, cc = i - r * kPerRow;
      *reinterpret_cast<u4*>(lds + r * (W + 4) + cc * 4) = v[q];
    }
  }
};

// 1. Local end state of each chunk, its decay, and the chunk's delta and
// cumulative log-decay (kept for the output kernel).
// With SEQ (packed documents), st_t is the chunk position of the latest
// document start at or before step t (-1 if none): step s <= t is in t's
// document exactly when s >= st_t, the carried state reaches t only when
// st_t = -1, the chunk's own end state sums the steps s >= st_end, and a chunk
// with a document start passes no older state on (decay 0).
template <int IO, int N, bool SEQ>
__global__ __launch_bounds__(kThreads) void ssd_state_kernel(
    int32_t seqlen, int32_t nheads, int32_t ngroups, int32_t nchunks, const typename Io<IO>::T* __restrict__ x,
    const typename Io<IO>::T* __restrict__ dt, const typename Io<IO>::T* __restrict__ Bm,
    const int32_t* __restrict__ seq_idx, const float* __restrict__ dt_bias, const float* __restrict__ A,
    float* __restrict__ states, float* __restrict__ decay, float* __restrict__ cs_out, float* __restrict__ dl_out,
    float* __restrict__ sg_out) {
  using T = typename Io<IO>::T;
  constexpr int kNT = N / 64;  // 16-row n-tiles per wave
  __shared__ float wgt[kQ], wsum[4], wmax[4], cs_last, st_last;
  __shared__ __align__(16) T bT[N][kTile + kPad];       // B^T of the s-tile: [n][s]
  __shared__ __align__(16) float wT[kP][kPitchT];  // (weight x)^T of the s-tile: [p][s], float32 or split
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, g16 = lane >> 4, c16 = lane & 15;
  const int32_t c = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int32_t grp = h / (nheads / ngroups);
  const int64_t t0 = static_cast<int64_t>(c) * kQ;
  const int valid = static_cast<int>(min(static_cast<int64_t>(kQ), seqlen - t0));
  const int64_t row0 = static_cast<int64_t>(b) * seqlen + t0;
  const int64_t ldB = static_cast<int64_t>(ngroups) * N, ldX = static_cast<int64_t>(nheads) * kP;
  const T* Bg = Bm + (row0 * ngroups + grp) * N;
  const T* Xg = x + row0 * ldX + h * kP;
  // first tile's loads, then delta and the cumulative log-decay of the chunk
  ColTile<IO, N> tb;
  typename WeightedTile<IO>::type tw;
  tb.load(Bg, ldB, min(kTile, valid), tid);
  tw.load(Xg, ldX, min(kTile, valid), tid);
  float delta = 0.0f;
  if (tid < valid) delta = softplus(Io<IO>::load(dt + (row0 + tid) * nheads + h) + dt_bias[h]);
  const float csv = block_scan(delta * A[h], wsum, tid);
  const int64_t bch = (static_cast<int64_t>(b) * nchunks + c) * nheads + h;
  cs_out[bch * kQ + tid] = csv;
  dl_out[bch * kQ + tid] = delta;
  float stv = -1.0f;
  if (SEQ) {
    const int64_t t = t0 + tid;  // a document starts at t when its id differs from step t-1's
    const bool start = tid < valid && t > 0 &&
                       seq_idx[static_cast<int64_t>(b) * seqlen + t] != seq_idx[static_cast<int64_t>(b) * seqlen + t - 1];
    stv = block_scan_max(start ? static_cast<float>(tid) : -1.0f, wmax, tid);  // exact: small integers
    sg_out[bch * kQ + tid] = stv;
  }
  if (tid == kQ - 1) {
    cs_last = csv;
    st_last = stv;
  }
  __syncthreads();
  const float cs_end = cs_last, st_end = st_last;
  wgt[tid] = (!SEQ || static_cast<float>(tid) >= st_end) ? exp2_hw((cs_end - csv) * kLog2e) * delta : 0.0f;
  f4 acc[kNT][4];
#pragma unroll
  for (int nt = 0; nt < kNT; ++nt)
#pragma unroll
    for (int pt = 0; pt < 4; ++pt) acc[nt][pt] = f4{0.0f, 0.0f, 0.0f, 0.0f};
  for (int s0 = 0; s0 < valid; s0 += kTile) {
    __syncthreads();  // previous tile's operands read; wgt written
    tb.store(&bT[0][0], tid);
    tw.store(&wT[0][0], &wgt[s0], tid);
    __syncthreads();
    if (s0 + kTile < valid) {  // the next tile's loads stay in flight over the products
      const int rows = min(kTile, valid - s0 - kTile);
      tb.load(Bg + (s0 + kTile) * ldB, ldB, rows, tid);
      tw.load(Xg + (s0 + kTile) * ldX, ldX, rows, tid);
    }
#pragma unroll
    for (int ks = 0; ks < kTile; ks += 32) {
      Frag<IO> a[kNT];
#pragma unroll
      for (int nt = 0; nt < kNT; ++nt) a[nt] = frag8(&bT[(wv * kNT + nt) * 16 + c16][ks + g16 * 8]);
#pragma unroll
      for (int pt = 0; pt < 4; ++pt) {
        const float* bq = &wT[pt * 16 + c16][ks + g16 * 8];
#pragma unroll
        for (int nt = 0; nt < kNT; ++nt) acc[nt][pt] = mma_state<IO>(a[nt], bq, acc[nt][pt]);
      }
    }
  }
  // lane holds S[n = tile*16 + 4 g16 + j][p = pt*16 + c16]: four consecutive n of the [p][n] layout
  float* out = states + bch * kP * N;
#pragma unroll
  for (int nt = 0; nt < kNT; ++nt)
#pragma unroll
    for (int pt = 0; pt < 4; ++pt)
      *reinterpret_cast<f4*>(out + (pt * 16 + c16) * N + (wv * kNT + nt) * 16 + g16 * 4) = acc[nt][pt];
  if (tid == 0) decay[bch] = (!SEQ || st_end < 0.0f) ? exp2_hw(cs_end * kLog2e) : 0.0f;
}

// 2. Carried states: each chunk's local state is replaced by the state that
// enters it; the last one out is the final state. A thread carries 8
// consecutive n of one row p. With SPLIT (bfloat16 io) the entering state is
// stored as the output kernel's matrix-core operand, hi and lo bfloat16 parts
// (split8) in the same 32 bytes, so that kernel's waves need not split it.
template <bool SPLIT>
__global__ __launch_bounds__(kThreads) void ssd_pass_kernel(int32_t nchunks, int32_t nheads, int32_t pn8,
                                                            const float* state_in, float* states,
                                                            const float* __restrict__ decay, float* state_out) {
  const int32_t e = static_cast<int32_t>(blockIdx.x) * kThreads + static_cast<int32_t>(threadIdx.x);
  if (e >= pn8) return;
  const int32_t h = blockIdx.y, b = blockIdx.z;
  const int64_t bh = static_cast<int64_t>(b) * nheads + h;
  f4 H0 = {0.0f, 0.0f, 0.0f, 0.0f}, H1 = H0;
  if (state_in) {
    const f4* src = reinterpret_cast<const f4*>(state_in) + (bh * pn8 + e) * 2;
    H0 = src[0];
    H1 = src[1];
  }
  for (int32_t c = 0; c < nchunks; ++c) {
    const int64_t bch = (static_cast<int64_t>(b) * nchunks + c) * nheads + h;
    f4* slot = reinterpret_cast<f4*>(states) + (bch * pn8 + e) * 2;
    const f4 S0 = slot[0], S1 = slot[1];
    if (SPLIT) {
      const Split sp = split8(H0, H1);
      u4* us = reinterpret_cast<u4*>(slot);
      us[0] = __builtin_bit_cast(u4, sp.hi.v);
      us[1] = __builtin_bit_cast(u4, sp.lo.v);
    } else {
      slot[0] = H0;
      slot[1] = H1;
    }
    const float d = decay[bch];
    H0 = d * H0 + S0;
    H1 = d * H1 + S1;
  }
  if (state_out) {
    f4* dst = reinterpret_cast<f4*>(state_out) + (bh * pn8 + e) * 2;
    dst[0] = H0;
    dst[1] = H1;
  }
}

// 3. Outputs of one 64-step tile of a chunk for HB heads of one group. G^T
// depends only on B and C, which the heads of a group share, so it is formed
// once per s-tile and applied to each head with that head's decay and x.
// Three waves per SIMD (the register budget that allows it: the bfloat16
// instances fit without spilling; the float32 d_state 128 one stays at two).
template <int IO, int N, bool SEQ, int HB>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(3))) void ssd_out_kernel(
    int32_t seqlen, int32_t nheads, int32_t ngroups, int32_t nchunks, const typename Io<IO>::T* __restrict__ x,
    const typename Io<IO>::T* __restrict__ Bm, const typename Io<IO>::T* __restrict__ Cm,
    const float* __restrict__ Dskip, const float* __restrict__ states, const float* __restrict__ cs_in,
    const float* __restrict__ dl_in, const float* __restrict__ sg_in, typename Io<IO>::T* __restrict__ y) {
  using T = typename Io<IO>::T;
  __shared__ __align__(16) float cs[HB][kQ];
  __shared__ __align__(16) float dl[HB][kQ];
  __shared__ __align__(16) float ex[HB][kQ];  // exp(cs_r - cs_s) delta_s, r the last step of s's 64-step tile
  __shared__ __align__(16) float sg[SEQ ? kQ : 4];  // latest document start at or before each step
  // B rows of the s-tile ([s][n]; at the end the output tile) and x^T of the
  // s-tile per head ([p][s]), carved from one region which, before the s-tile
  // loop, holds the two slice buffers of the carried state (kSW columns each)
  constexpr int kBsBytes = kTile * (N + kPad) * static_cast<int>(sizeof(T));
  constexpr int kXtBytes = HB * kP * kPitchT * static_cast<int>(sizeof(T));
  constexpr int kSW = 2 * kP * (64 + 4) * 4 <= kBsBytes + kXtBytes ? 64 : 32;
  constexpr int kSlBytes = kP * (kSW + 4) * 4;
  constexpr int kRegion = kBsBytes + kXtBytes > 2 * kSlBytes ? kBsBytes + kXtBytes : 2 * kSlBytes;
  __shared__ __align__(16) unsigned char region[kRegion];
  auto& bS = *reinterpret_cast<T(*)[kTile][N + kPad]>(region);
  auto& xT = *reinterpret_cast<T(*)[HB][kP][kPitchT]>(region + kBsBytes);
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, g16 = lane >> 4, c16 = lane & 15;
  // Workgroups are dispatched to the 8 XCDs round-robin by linear id, and each
  // XCD has its own L2. The four t-tiles of one (b, chunk, head pair) read the
  // same carried state and x tiles, so logical ids are assigned in
  // contiguous ranges per XCD: those four run on one XCD, close in time.
  int32_t c, tt, hp, b;
  {
    const int32_t gx = static_cast<int32_t>(gridDim.x), gy = static_cast<int32_t>(gridDim.y);
    const int32_t total = gx * gy * static_cast<int32_t>(gridDim.z);
    const int32_t lin = static_cast<int32_t>(blockIdx.x) + gx * (static_cast<int32_t>(blockIdx.y) +
                                                                  gy * static_cast<int32_t>(blockIdx.z));
    const int32_t q = total >> 3, r = total & 7, xcd = lin & 7, i = lin >> 3;
    int32_t w = xcd * q + min(xcd, r) + i;  // logical id: t-tile fastest, then chunk, head pair, batch row
    tt = w & 3;
    w >>= 2;
    c = w % nchunks;
    w /= nchunks;
    hp = w % gy;
    b = w / gy;
  }
  const int32_t h0 = hp * HB;  // heads h0 .. h0+HB-1
  const int32_t grp = h0 / (nheads / ngroups);  // the host keeps the HB heads in one group
  const int64_t t0 = static_cast<int64_t>(c) * kQ;
  const int valid = static_cast<int>(min(static_cast<int64_t>(kQ), seqlen - t0));
  const int tb = tt * kTile;  // first step of the t-tile in the chunk
  if (tb >= valid) return;    // the whole workgroup, before any barrier
  const int64_t row0 = static_cast<int64_t>(b) * seqlen + t0;
  const int64_t ldB = static_cast<int64_t>(ngroups) * N, ldX = static_cast<int64_t>(nheads) * kP;
  const T* Bg = Bm + (row0 * ngroups + grp) * N;
  const T* Xg = x + row0 * ldX + h0 * kP;  // head h0 + hh at Xg + hh * kP
  const int64_t bch0 = (static_cast<int64_t>(b) * nchunks + c) * nheads + h0;
  // every first load is issued before the first use (loads complete in order).
  // The lane's C fragments (row t = tb + 16 wv + c16, 8 consecutive n per
  // K-step) are contiguous in memory and the same for every product below, so
  // they stay in registers (rows past the end read row 0 and are zeroed).
  constexpr int kKS = N / 32;
  Frag<IO> cf[kKS];
  {
    const int tr = tb + wv * 16 + c16;
    const T* crow = Cm + ((row0 + (tr < valid ? tr : 0)) * ngroups + grp) * N + g16 * 8;
#pragma unroll
    for (int k = 0; k < kKS; ++k) cf[k] = frag8(crow + 32 * k);
    if (tr >= valid) {
#pragma unroll
      for (int k = 0; k < kKS; ++k) cf[k] = frag_zero<IO>();
    }
  }
  float csv[HB], dlv[HB];
#pragma unroll
  for (int hh = 0; hh < HB; ++hh) {
    csv[hh] = cs_in[(bch0 + hh) * kQ + tid];
    dlv[hh] = dl_in[(bch0 + hh) * kQ + tid];
  }
  const float sgv = SEQ ? sg_in[bch0 * kQ + tid] : -1.0f;  // the same for every head
  RowTile<IO, N> tbs;  // s-tile 0, in flight over the carried-state product
  ColTile<IO, kP, kPitchT> txs[HB];
  tbs.load(Bg, ldB, min(kTile, valid), tid);
#pragma unroll
  for (int hh = 0; hh < HB; ++hh) txs[hh].load(Xg + hh * kP, ldX, min(kTile, valid), tid);
#pragma unroll
  for (int hh = 0; hh < HB; ++hh) {
    cs[hh][tid] = csv[hh];
    dl[hh][tid] = dlv[hh];
    // a 64-step tile is one wave, so its last step's cs is lane 63's
    const float csr = __shfl(csv[hh], 63, 64);
    ex[hh][tid] = exp2_hw(fminf((csr - csv[hh]) * kLog2e, 0.0f)) * dlv[hh];
  }
  if (SEQ) sg[tid] = sgv;

  // carried state: Y[t][p] = exp(cs_t) sum_n C[t][n] S_in[p][n], S_in staged
  // through LDS in kSW-column slices, head after head (for bfloat16 io it
  // arrives split into hi and lo parts): two buffers over the tile region
  // (not yet used), two slices in flight, one barrier per slice
  f4 acc[HB][4];
  {
    constexpr int kPer = N / kSW, kIt = HB * kPer;
    float* const buf0 = reinterpret_cast<float*>(region);
    float* const buf1 = reinterpret_cast<float*>(region + kSlBytes);
    StateSlice<kSW> sa, sb;  // the slices of even and of odd iterations
    sa.load(states + bch0 * kP * N, N, 0, tid);
    if (kIt > 1) sb.load(states + (bch0 + 1 / kPer) * kP * N, N, (1 % kPer) * kSW, tid);
#pragma unroll
    for (int hh = 0; hh < HB; ++hh) {
#pragma unroll
      for (int pt = 0; pt < 4; ++pt) acc[hh][pt] = f4{0.0f, 0.0f, 0.0f, 0.0f};
    }
#pragma unroll
    for (int it = 0; it < kIt; ++it) {
      const int hh = it / kPer, k0 = (it % kPer) * kSW;
      float* const bf = (it & 1) ? buf1 : buf0;
      // every wave passed the previous barrier, so it is done with the slice
      // of iteration it - 2 in this buffer
      if (it & 1) {
        sb.store(bf, tid);
      } else {
        sa.store(bf, tid);
      }
      __syncthreads();  // slice it visible (first pass: cs, dl, ex, sg written)
      if (it + 2 < kIt) {
        const float* g = states + (bch0 + (it + 2) / kPer) * kP * N;
        if (it & 1) {
          sb.load(g, N, ((it + 2) % kPer) * kSW, tid);
        } else {
          sa.load(g, N, ((it + 2) % kPer) * kSW, tid);
        }
      }
#pragma unroll
      for (int kk = 0; kk < kSW; kk += 32) {
#pragma unroll
        for (int pt = 0; pt < 4; ++pt)
          acc[hh][pt] = mma_state<IO>(cf[(k0 + kk) / 32], bf + (pt * 16 + c16) * (kSW + 4) + kk + g16 * 8,
                                      acc[hh][pt]);
      }
    }
    f4 sg4 = {-1.0f, -1.0f, -1.0f, -1.0f};
    if (SEQ) sg4 = *reinterpret_cast<const f4*>(&sg[tb + wv * 16 + g16 * 4]);
#pragma unroll
    for (int hh = 0; hh < HB; ++hh) {
      const f4 cs4 = *reinterpret_cast<const f4*>(&cs[hh][tb + wv * 16 + g16 * 4]);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float e = sg4[j] < 0.0f ? exp2_hw(cs4[j] * kLog2e) : 0.0f;  // no document start up to t
#pragma unroll
        for (int pt = 0; pt < 4; ++pt) acc[hh][pt][j] *= e;
      }
    }
  }

  // intra-chunk: s-tiles up to the own one
  const int tpos = tb + wv * 16 + c16;  // this lane's step as the column of G^T / row of G
  float cst[HB];
#pragma unroll
  for (int hh = 0; hh < HB; ++hh) cst[hh] = cs[hh][tpos];
  // first step of t's document in this chunk (0 when it began earlier) and
  // the tile-relative bounds of the diagonal mask: keep lo <= s <= t
  const int lo = SEQ ? max(static_cast<int>(sg[tpos]), 0) : 0;
  for (int sb = 0; sb <= tb; sb += kTile) {
    __syncthreads();  // previous s-tile's operands read
    tbs.store(&bS[0][0], tid);
#pragma unroll
    for (int hh = 0; hh < HB; ++hh) txs[hh].store(&xT[hh][0][0], tid);
    __syncthreads();
    if (sb + kTile <= tb) {  // the next s-tile's loads stay in flight over the products
      const int rows = min(kTile, valid - sb - kTile);
      tbs.load(Bg + (sb + kTile) * ldB, ldB, rows, tid);
#pragma unroll
      for (int hh = 0; hh < HB; ++hh) txs[hh].load(Xg + (sb + kTile) * ldX + hh * kP, ldX, rows, tid);
    }
    // G^T[s][t] = sum_n B[s][n] C[t][n]: lane holds s = si*16 + 4 g16 + j, t = tpos
    f4 gt[4];
#pragma unroll
    for (int si = 0; si < 4; ++si) {
      gt[si] = f4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int ks = 0; ks < N; ks += 32)
        gt[si] = mma(frag8(&bS[si * 16 + c16][ks + g16 * 8]), cf[ks / 32], gt[si]);
    }
    // On the diagonal tile: causal mask (and same document), shared by the
    // heads, G^T zeroed past the diagonal; below it cs_t <= cs_s, so each
    // head's exponent is clamped at 0 (it only differs from that by rounding
    // in the scan) and the factor stays finite where G^T was zeroed.
    // On an earlier tile every s < t, and exp(cs_t - cs_s) = exp(cs_t - cs_r)
    // exp(cs_r - cs_s) with r the tile's last step, both exponents <= 0: one
    // exp per lane and head times the table ex (only the document mask left).
    const bool diag = sb == tb;  // wave-uniform
    if (diag || SEQ) {
#pragma unroll
      for (int si = 0; si < 4; ++si) {
        const int s4 = sb + si * 16 + g16 * 4;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const bool keep = (!diag || s4 + j <= tpos) && (!SEQ || s4 + j >= lo);
          gt[si][j] = keep ? gt[si][j] : 0.0f;
        }
      }
    }
#pragma unroll
    for (int hh = 0; hh < HB; ++hh) {
      // decay exp(cs_t - cs_s) and delta_s of this head, in float32
      f4 gm[4];
      if (diag) {
#pragma unroll
        for (int si = 0; si < 4; ++si) {
          const int s4 = sb + si * 16 + g16 * 4;
          const f4 cs4 = *reinterpret_cast<const f4*>(&cs[hh][s4]);
          const f4 dl4 = *reinterpret_cast<const f4*>(&dl[hh][s4]);
#pragma unroll
          for (int j = 0; j < 4; ++j)
            gm[si][j] = gt[si][j] * (exp2_hw(fminf((cst[hh] - cs4[j]) * kLog2e, 0.0f)) * dl4[j]);
        }
      } else {
        const float et = exp2_hw(fminf((cst[hh] - cs[hh][sb + kTile - 1]) * kLog2e, 0.0f));
#pragma unroll
        for (int si = 0; si < 4; ++si) {
          const f4 ex4 = *reinterpret_cast<const f4*>(&ex[hh][sb + si * 16 + g16 * 4]);
          gm[si] = gt[si] * (ex4 * et);
        }
      }
      // Y[t][p] += sum_s G[t][s] x[s][p], K order: slots 0-3 from tile 2m, 4-7 from tile 2m+1
#pragma unroll
      for (int m = 0; m < 2; ++m) {
#pragma unroll
        for (int pt = 0; pt < 4; ++pt) {
          const T* row = &xT[hh][pt * 16 + c16][0];
          acc[hh][pt] = mma_f32a<IO>(gm[2 * m], gm[2 * m + 1],
                                     frag44(row + 32 * m + 4 * g16, row + 32 * m + 16 + 4 * g16), acc[hh][pt]);
        }
      }
    }
  }

  // D skip (x of the own t-tile is the last staged x^T) and the output tiles,
  // head after head, through LDS (over bS, no longer read), stored as whole
  // 128-byte rows
  T* yt = &bS[0][0];  // [64][kP + kPad]
  static_assert(sizeof(bS) >= kTile * (kP + kPad) * sizeof(T), "output tile must fit");
  constexpr int kVec = 16 / static_cast<int>(sizeof(T));
  constexpr int kPer = kP / kVec;
  const int rows = min(kTile, valid - tb);
  // the lane's row and column bits, derived afresh from the thread id (the
  // empty asm hides the earlier ones, which would otherwise be kept in a
  // register, or spilled, across every loop above)
  int otid = static_cast<int>(threadIdx.x);
  asm volatile("" : "+v"(otid));
  const int orow = (otid >> 6) * 16 + ((otid >> 4) & 3) * 4, ocol = otid & 15;
#pragma unroll
  for (int hh = 0; hh < HB; ++hh) {
    const float dsk = Dskip[h0 + hh];
    __syncthreads();  // every wave's reads of bS (or of the previous head's tile) are done
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int tl = orow + j;  // row in the t-tile: 16 wv + 4 g16 + j
#pragma unroll
      for (int pt = 0; pt < 4; ++pt) {
        const int p = pt * 16 + ocol;
        Io<IO>::store(yt + tl * (kP + kPad) + p, fmaf(dsk, Io<IO>::cvt(xT[hh][p][tl]), acc[hh][pt][j]));
      }
    }
    __syncthreads();
    T* yg = y + (row0 + tb) * ldX + (h0 + hh) * kP;
    for (int i = tid; i < kTile * kPer; i += kThreads) {
      const int r = i / kPer, cc = i - r * kPer;
      if (r < rows)
        *reinterpret_cast<u4*>(yg + r * ldX + cc * kVec) = *reinterpret_cast<const u4*>(yt + r * (kP + kPad) + cc * kVec);
    }
  }
}

// One token per batch row (niverel-mamba 0.1.0 PKG-INFO, "Autoregressive
// decoding": the step returns the new state). A state row S[b][h][p][0..N) is
// handled by N/4 lanes holding four consecutive states each (one 16-byte
// access per lane, whole rows per wave); the readout sum over n is a shuffle
// reduction over those lanes. Memory-bound: the state is read and written once.
template <int IO, int N>
__global__ __launch_bounds__(kThreads) void ssd_step_kernel(int32_t rows, int32_t nheads, int32_t ngroups,
                                                            const typename Io<IO>::T* __restrict__ x,
                                                            const typename Io<IO>::T* __restrict__ dt,
                                                            const typename Io<IO>::T* __restrict__ Bm,
                                                            const typename Io<IO>::T* __restrict__ Cm,
                                                            const float* __restrict__ dt_bias, const float* __restrict__ A,
                                                            const float* __restrict__ Dskip, const float* state_in,
                                                            typename Io<IO>::T* __restrict__ y, float* state_out) {
  constexpr int kLanes = N / 4;  // lanes per state row (32 or 16)
  // rows * kLanes lanes can pass 2^31 (and a dispatch dimension's 2^32): the
  // workgroups are numbered over a 2D grid and the lane index is 64-bit
  const int64_t gid = (static_cast<int64_t>(blockIdx.y) * gridDim.x + blockIdx.x) * kThreads + threadIdx.x;
  const int64_t row = gid / kLanes;  // row = (b * nheads + h) * 64 + p
  const int32_t q = static_cast<int32_t>(threadIdx.x) % kLanes;
  const bool live = row < rows;
  const int32_t r = live ? static_cast<int32_t>(row) : rows - 1;  // idle lanes mirror the last row, store nothing
  const int32_t bh = r / kP, b = bh / nheads, h = bh - b * nheads;
  const int32_t g = h / (nheads / ngroups);
  const float delta = softplus(Io<IO>::load(dt + bh) + dt_bias[h]);
  const float decay = exp2_hw(delta * A[h] * kLog2e);
  const float xv = Io<IO>::load(x + r);
  const int64_t bn = (static_cast<int64_t>(b) * ngroups + g) * N + q * 4;
  float bv[4], cv[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    bv[k] = Io<IO>::load(Bm + bn + k);
    cv[k] = Io<IO>::load(Cm + bn + k);
  }
  const int64_t so = static_cast<int64_t>(r) * N + q * 4;
  const f4 s0 = __builtin_nontemporal_load(reinterpret_cast<const f4*>(state_in + so));
  const float dx = delta * xv;
  f4 s1;
  float part = 0.0f;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    s1[k] = fmaf(decay, s0[k], dx * bv[k]);
    part = fmaf(cv[k], s1[k], part);
  }
  if (live) __builtin_nontemporal_store(s1, reinterpret_cast<f4*>(state_out + so));
#pragma unroll
  for (int o = kLanes / 2; o > 0; o >>= 1) part += __shfl_xor(part, o, kLanes);
  if (live && q == 0) Io<IO>::store(y + r, fmaf(Dskip[h], xv, part));
}

template <int IO, int N>
hipError_t launch_step_typed(const SsdCall& c) {
  using T = typename Io<IO>::T;
  const int32_t rows = c.batch * c.nheads * kP;
  // at most 2^22 workgroups along x (a dispatch dimension counts its
  // work-items in 32 bits), the rest along y
  const int64_t blocks = (static_cast<int64_t>(rows) * (N / 4) + kThreads - 1) / kThreads;
  const int64_t gx = blocks < (int64_t{1} << 22) ? blocks : (int64_t{1} << 22);
  hipLaunchKernelGGL((ssd_step_kernel<IO, N>),
                     dim3(static_cast<unsigned>(gx), static_cast<unsigned>((blocks + gx - 1) / gx)), dim3(kThreads), 0, c.stream, rows, c.nheads, c.ngroups, static_cast<const T*>(c.x),
                     static_cast<const T*>(c.dt), static_cast<const T*>(c.B), static_cast<const T*>(c.C), c.dt_bias,
                     c.A, c.D, c.state_in, static_cast<T*>(c.y), c.state_out);
  return hipGetLastError();
}

template <int IO, int N, bool SEQ, int HB>
void launch_out(const SsdCall& c, int32_t nchunks, const float* states, const float* cs, const float* dl,
                const float* sg) {
  using T = typename Io<IO>::T;
  hipLaunchKernelGGL((ssd_out_kernel<IO, N, SEQ, HB>), dim3(nchunks * 4, c.nheads / HB, c.batch), dim3(kThreads), 0,
                     c.stream, c.seqlen, c.nheads, c.ngroups, nchunks, static_cast<const T*>(c.x),
                     static_cast<const T*>(c.B), static_cast<const T*>(c.C), c.D, states, cs, dl, sg,
                     static_cast<T*>(c.y));
}

template <int IO, int N, bool SEQ>
hipError_t launch_typed(const SsdCall& c) {
  using T = typename Io<IO>::T;
  const int32_t nchunks = (c.seqlen + kQ - 1) / kQ;
  const SsdWs w = ssd_ws_layout(c.batch, c.seqlen, c.nheads, c.d_state);
  float* states = c.workspace + w.states;
  float* decay = c.workspace + w.decay;
  float* cs = c.workspace + w.cs;
  float* dl = c.workspace + w.dl;
  float* sg = c.workspace + w.sg;
  hipLaunchKernelGGL((ssd_state_kernel<IO, N, SEQ>), dim3(nchunks, c.nheads, c.batch), dim3(kThreads), 0, c.stream,
                     c.seqlen, c.nheads, c.ngroups, nchunks, static_cast<const T*>(c.x), static_cast<const T*>(c.dt),
                     static_cast<const T*>(c.B), c.seq_idx, c.dt_bias, c.A, states, decay, cs, dl, sg);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int32_t pn8 = kP * N / 8;
  hipLaunchKernelGGL(ssd_pass_kernel<IO == 1>, dim3((pn8 + kThreads - 1) / kThreads, c.nheads, c.batch),
                     dim3(kThreads), 0, c.stream, nchunks, c.nheads, pn8, c.state_in, states, decay, c.state_out);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  // bfloat16: two heads of a group per workgroup share G^T (float32 keeps one:
  // its operands take twice the registers)
  if (IO == 1 && (c.nheads / c.ngroups) % 2 == 0)
    launch_out<IO, N, SEQ, IO == 1 ? 2 : 1>(c, nchunks, states, cs, dl, sg);
  else
    launch_out<IO, N, SEQ, 1>(c, nchunks, states, cs, dl, sg);
  return hipGetLastError();
}

}  // namespace

SsdWs ssd_ws_layout(int32_t batch, int32_t seqlen, int32_t nheads, int32_t d_state) {
  SsdWs w{};
  const size_t nchunks = (static_cast<size_t>(seqlen) + kQ - 1) / kQ;
  const size_t bch = static_cast<size_t>(batch) * nchunks * nheads;
  w.states = 0;
  w.decay = bch * kP * d_state;
  w.cs = w.decay + ((bch + 63) / 64) * 64;
  w.dl = w.cs + bch * kQ;
  w.sg = w.dl + bch * kQ;
  w.total = w.sg + bch * kQ;
  return w;
}

hipError_t launch_ssd_step(const SsdCall& c) {
  if (c.io_dtype == 0) return c.d_state == 64 ? launch_step_typed<0, 64>(c) : launch_step_typed<0, 128>(c);
  return c.d_state == 64 ? launch_step_typed<1, 64>(c) : launch_step_typed<1, 128>(c);
}

template <bool SEQ>
hipError_t launch_ssd_seq(const SsdCall& c) {
  if (c.io_dtype == 0) return c.d_state == 64 ? launch_typed<0, 64, SEQ>(c) : launch_typed<0, 128, SEQ>(c);
  return c.d_state == 64 ? launch_typed<1, 64, SEQ>(c) : launch_typed<1, 128, SEQ>(c);
}

hipError_t launch_ssd(const SsdCall& c) { return c.seq_idx ? launch_ssd_seq<true>(c) : launch_ssd_seq<false>(c); }

}  // namespace mscan
