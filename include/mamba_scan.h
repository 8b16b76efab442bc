/*
 * mamba_scan.h -- C ABI of the MI355X (gfx950) selective-scan library
 * libmamba_scan.so.
 *
 * The operation (calm-mamba 0.1.4 PKG-INFO, "Architecture" / "Mamba operator",
 * steps 2, 4 (the softplus), 5 and 6) for every batch row b and channel d:
 *
 *   xc[t]    = SiLU(conv_b[d] + sum_{k<4} conv_w[d][k] * xw[t-3+k])
 *              (causal depthwise conv1d, kernel 4, xw = conv history ++ x;
 *              tap 3 multiplies the newest token)
 *   delta[t] = softplus(dt[t] + dt_bias[d])
 *   h[t][n]  = exp(delta[t] * A[d][n]) * h[t-1][n] + delta[t] * B[t][n] * xc[t]
 *   y[t]     = (sum_n C[t][n] * h[t][n] + D[d] * xc[t]) * SiLU(z[t])
 *
 * The in/x/dt/out projections (steps 1, 3, the dt matmul and 7) are outside
 * this library. Conv and SSM states come back for resume, and the one-token
 * step is functional: it maps (states, token) to (output, new states), as the
 * decoding contract in niverel-mamba 0.1.0 PKG-INFO ("Autoregressive
 * decoding") states it.
 *
 * Conventions shared by every entry point
 *  - Every array pointer is a DEVICE pointer owned by the caller; the library
 *    allocates no device memory and keeps no state between calls except a
 *    per-thread last-error string, a global successful-call counter and the
 *    fixed device scratch of mamba_scan_fwd_noalloc.
 *  - Arrays are dense and row-major with the shapes given below.
 *    "io" arrays hold io_dtype elements (MAMBA_F32: float, MAMBA_BF16:
 *    bfloat16 stored as uint16); parameters and states are always float32.
 *  - Calls are asynchronous on `stream` (a hipStream_t; NULL = the default
 *    stream). The return value reports argument validation and the launch
 *    only; faults during execution surface at the caller's next
 *    synchronisation. Inputs must stay valid until the stream has run the
 *    call.
 *  - Validation runs before any HIP call, in this order: dims (MAMBA_ERR_SHAPE),
 *    io_dtype (MAMBA_ERR_DTYPE), required pointers (MAMBA_ERR_NULL),
 *    element alignment (MAMBA_ERR_ALIGN), overlaps (MAMBA_ERR_ALIAS),
 *    workspace size (MAMBA_ERR_WORKSPACE), then the device (MAMBA_ERR_DEVICE:
 *    no visible gfx950 device, or a failed launch). On any error nothing is
 *    launched and mamba_scan_last_error() says why. There is no CPU or other
 *    fallback: an explicit request either runs as asked or fails with a
 *    status (niverel-mamba 0.1.0 PKG-INFO, "No silent fallback"), and a call
 *    with no usable gfx950 device fails clearly with MAMBA_ERR_DEVICE rather
 *    than running elsewhere (openfluke "Apple Mamba stress test", "Build
 *    requirements": a missing backend fails clearly).
 *  - NaN and Inf propagate; nothing is clamped. Results are deterministic:
 *    the same inputs give bit-identical outputs on every run.
 *  - Precision: all arithmetic is float32; y is rounded to io_dtype
 *    (round-to-nearest-even for bfloat16). The exponential, logarithm and
 *    reciprocal come from the hardware approximations, so results are not
 *    bit-identical to a float64 evaluation (agreement is checked to a
 *    relative 1e-4 for float32 io and 2e-2 for bfloat16 io).
 */
#ifndef MAMBA_SCAN_H
#define MAMBA_SCAN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MAMBA_SCAN_ABI_VERSION 1

typedef enum { MAMBA_F32 = 0, MAMBA_BF16 = 1 } mamba_io_dtype;

typedef enum {
  MAMBA_OK = 0,
  MAMBA_ERR_NULL = 1,      /* a required pointer is NULL                         */
  MAMBA_ERR_SHAPE = 2,     /* a dim < 1, d_conv != 4, d_state not 8 or 16, or too large */
  MAMBA_ERR_DTYPE = 3,     /* io_dtype is not MAMBA_F32 / MAMBA_BF16              */
  MAMBA_ERR_ALIGN = 4,     /* a pointer is not aligned to its element size        */
  MAMBA_ERR_ALIAS = 5,     /* an output overlaps an input it may not overlap      */
  MAMBA_ERR_WORKSPACE = 6, /* workspace NULL or smaller than required             */
  MAMBA_ERR_DEVICE = 7     /* no gfx950 device current, or the launch failed      */
} mamba_status;

/* MAMBA_SCAN_ABI_VERSION of the loaded library. */
int mamba_scan_abi_version(void);

/* Static name of a status code ("MAMBA_OK", ...); "unknown status" otherwise. */
const char* mamba_scan_status_str(int status);

/* Detail of the last failed call on this thread ("" after a success). The
   string is owned by the library and valid until the thread's next call. */
const char* mamba_scan_last_error(void);

/* Number of calls of any compute entry point of this library, over the
   whole process, that passed validation and launched their kernels: the
   count of successful native calls that a run's metadata records (openfluke
   "Apple Mamba stress test", "What the results mean"), so that a harness can
   tell native execution from any other path. */
uint64_t mamba_scan_call_count(void);

/* Bytes of device workspace mamba_scan_fwd (and mamba_scan_fwd_seq,
   mamba_scan_fwd_ckpt) needs for this shape and dtype (0 when the sequence is
   not split into chunks). Returns 0 for shapes that mamba_scan_fwd would
   reject. A pure function of the arguments. It takes io_dtype beside the
   shape because the kernel plan, and hence the chunk split, is chosen per
   io dtype (the split's own arrays are float32 either way). */
size_t mamba_scan_fwd_workspace_bytes(int32_t batch, int32_t seqlen, int32_t d_inner,
                                      int32_t d_state, int32_t io_dtype);

/*
 * Full-sequence prefill (calm-mamba 0.1.4 PKG-INFO, "Mamba operator", steps
 * 2, 4, 5, 6 over t = 0 .. seqlen-1).
 *
 *   x, dt, z        [batch][seqlen][d_inner]  io   (dt is the projection output
 *                                                   WITHOUT dt_bias)
 *   B, C            [batch][seqlen][d_state]  io   (shared by all channels)
 *   conv_w          [d_inner][d_conv]         f32  (tap d_conv-1 = newest x)
 *   conv_b, dt_bias, D   [d_inner]            f32
 *   A               [d_inner][d_state]        f32  (A = -exp(A_log), given)
 *   conv_state_in   [batch][d_inner][d_conv-1] f32, index 0 = oldest x; NULL = zeros
 *   ssm_state_in    [batch][d_inner][d_state]  f32; NULL = zeros
 *   y               [batch][seqlen][d_inner]  io   (output; must not overlap any input)
 *   conv_state_out  as conv_state_in; NULL = not written. It receives the last
 *                   d_conv-1 entries of (conv history ++ x) as exact copies.
 *   ssm_state_out   as ssm_state_in; NULL = not written; h after the last token.
 *                   Each state output may be exactly the matching input
 *                   (in-place update) or disjoint from every input; a partial
 *                   overlap is MAMBA_ERR_ALIAS.
 *   workspace       device scratch of at least
 *                   mamba_scan_fwd_workspace_bytes(...) bytes (NULL allowed when
 *                   that is 0); contents on entry are ignored. The call uses it
 *                   until the stream has run the call, so concurrent calls need
 *                   distinct workspaces.
 *   d_conv must be 4 and d_state 8 or 16; batch, seqlen, d_inner >= 1,
 *   d_inner <= 2^24 (a stage's rows are addressed through 32-bit buffer
 *   ranges), and the element counts must fit in int32 per tensor row index
 *   maths (batch*seqlen*max(d_inner, d_state) < 2^31).
 */
int mamba_scan_fwd(int32_t batch, int32_t seqlen, int32_t d_inner, int32_t d_state,
                   int32_t d_conv, int32_t io_dtype, const void* x, const void* dt, const void* z,
                   const void* B, const void* C, const float* conv_w, const float* conv_b,
                   const float* dt_bias, const float* D, const float* A,
                   const float* conv_state_in, const float* ssm_state_in, void* y,
                   float* conv_state_out, float* ssm_state_out, void* workspace,
                   size_t workspace_bytes, void* stream);

/*
 * Prefill over packed documents (niverel-mamba 0.1.0 PKG-INFO, "seq_idx
 * strict reset"): as mamba_scan_fwd, plus
 *
 *   seq_idx         [batch][seqlen] int32 document ids (required, 4-byte aligned)
 *
 * Wherever seq_idx[b][t] differs from seq_idx[b][t-1] (t >= 1) a new document
 * starts: the conv history and the SSM state of row b are zero before t, so
 * each document's outputs equal a separate mamba_scan_fwd over it from zero
 * states (the first document of a row starts from conv_state_in /
 * ssm_state_in). Ids are only compared for equality with the previous step;
 * they need not be increasing, and boundaries may fall anywhere. The states
 * written are those at the end of each row's last document. Same workspace,
 * validation, aliasing and error behaviour as mamba_scan_fwd (seq_idx counts
 * as an input).
 */
int mamba_scan_fwd_seq(int32_t batch, int32_t seqlen, int32_t d_inner, int32_t d_state,
                       int32_t d_conv, int32_t io_dtype, const void* x, const void* dt, const void* z,
                       const void* B, const void* C, const int32_t* seq_idx, const float* conv_w,
                       const float* conv_b, const float* dt_bias, const float* D, const float* A,
                       const float* conv_state_in, const float* ssm_state_in, void* y,
                       float* conv_state_out, float* ssm_state_out, void* workspace,
                       size_t workspace_bytes, void* stream);

/*
 * Prefill from the activated conv output (calm-mamba 0.1.4 PKG-INFO,
 * "Mamba operator", steps 4, 5 and 6 over t = 0 .. seqlen-1, with step 2's
 * result given): for a caller that has already computed
 *   xc[b][t][d] = SiLU(conv_b[d] + sum_k conv_w[d][k] * xw[t-3+k])
 * (a whole mixer layer does, because x_proj consumes xc), the scan, readout,
 * D skip and gate of mamba_scan_fwd, without recomputing the conv.
 *
 *   xc              [batch][seqlen][d_inner]  io   (replaces x)
 *   B, C            rows of d_state io elements, row (b, t) starting
 *                   (b * seqlen + t) * bc_stride elements past the pointer:
 *                   bc_stride = d_state is the contiguous [batch][seqlen][d_state]
 *                   of mamba_scan_fwd; a larger stride reads B and C in place
 *                   from a wider row, such as x_proj's output [tokens][dt_rank +
 *                   2 * d_state]. d_state <= bc_stride <= 2^24, batch * seqlen *
 *                   bc_stride < 2^31 (else MAMBA_ERR_SHAPE).
 *   dt, z, dt_bias, D, A, ssm_state_in, y, ssm_state_out, workspace:
 *                   as mamba_scan_fwd (the same workspace query applies)
 * There are no conv weights and no conv states: the caller keeps the conv
 * history. Same validation, aliasing rules (B and C cover the elements from
 * their first to the end of their last row), statuses and determinism as
 * mamba_scan_fwd; y equals mamba_scan_fwd's up to the rounding of the caller's
 * xc (bit for bit when xc holds the values mamba_scan_fwd computes internally,
 * which float32 io can carry).
 */
int mamba_scan_fwd_xc(int32_t batch, int32_t seqlen, int32_t d_inner, int32_t d_state, int32_t io_dtype,
                      const void* xc, const void* dt, const void* z, const void* B, const void* C, int32_t bc_stride,
                      const float* dt_bias, const float* D, const float* A, const float* ssm_state_in, void* y,
                      float* ssm_state_out, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Prefill from the activated conv output with dt_proj inside (calm-mamba
 * 0.1.4 PKG-INFO, "Mamba operator", step 4's projection fused with steps 4-6
 * around the scan, for a prefilling layer): as mamba_scan_fwd_xc, except that
 * dt is not passed; it is computed per (b, t, d) as
 *   dt[b][t][d] = sum_k dt_low[b][t][k] * w_dt[d][k],  k < dt_rank,
 * in float32 on the matrix cores and rounded to io_dtype (the value a layer
 * storing dt in that dtype would read back), then softplus(dt + dt_bias) as
 * usual.
 *
 *   dt_low   rows of dt_rank io elements, row (b, t) starting
 *            (b * seqlen + t) * dtl_stride elements past the pointer (x_proj's
 *            output [tokens][dt_rank + 2 * d_state] read in place); the
 *            pointer and dtl_stride * sizeof(io element) 4-byte aligned
 *   w_dt     [d_inner][dt_rank] io (dt_proj's weight, torch Linear layout)
 *   z        rows of d_inner io elements, row (b, t) starting
 *            (b * seqlen + t) * z_stride elements past the pointer: z_stride =
 *            d_inner is the contiguous layout; a larger stride reads z in
 *            place from a wider row, such as in_proj's output [tokens][2 *
 *            d_inner] (x, then z); d_inner <= z_stride <= 2^24
 *   d_state = 16; dt_rank a multiple of 8 in [8, 64]; dt_rank <= dtl_stride
 *   <= 2^24; batch * seqlen * dtl_stride and batch * seqlen * z_stride below
 *   2^31 (else MAMBA_ERR_SHAPE or MAMBA_ERR_ALIGN).
 * The other arguments, the workspace query (mamba_scan_fwd_workspace_bytes),
 * validation (dt_low and w_dt count as inputs in the aliasing rules, z covers
 * the elements from its first to the end of its last row), statuses and
 * determinism are those of mamba_scan_fwd_xc.
 */
int mamba_scan_fwd_xc_dtproj(int32_t batch, int32_t seqlen, int32_t d_inner, int32_t d_state, int32_t dt_rank,
                             int32_t io_dtype, const void* xc, const void* dt_low, int32_t dtl_stride,
                             const void* w_dt, const void* z, int32_t z_stride, const void* B, const void* C,
                             int32_t bc_stride, const float* dt_bias, const float* D, const float* A,
                             const float* ssm_state_in, void* y, float* ssm_state_out, void* workspace,
                             size_t workspace_bytes, void* stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the prefill
 * of mamba_scan_fwd, with the workspace taken from a fixed device array inside
 * the library instead of from the caller.
 *
 *   Every argument except the absent workspace pair is that of mamba_scan_fwd,
 *   with the same layouts, validation, aliasing rules and statuses.
 *   The array holds MAMBA_SCAN_NOALLOC_SCRATCH_BYTES (8 MiB). That is more
 *   than the workspace of any shape mamba_scan_fwd accepts: the sequence is
 *   split only until the launch reaches a fixed number of waves, which keeps
 *   the chunk summaries and state copies below about 7.3 MiB. A shape that
 *   needed more would be refused with MAMBA_ERR_WORKSPACE before any HIP
 *   call. The call itself allocates
 *   nothing (no hipMalloc, hipFree or allocating library routine); each
 *   device the library runs on holds its own copy of the array until the
 *   process ends.
 *   All calls on one device share that device's array, which keeps the last
 *   call's contents (nothing in it needs to start at zero). Calls that overlap
 *   in time on one device (different streams, or threads without ordering
 *   between them) race on it and give undefined results; calls ordered on
 *   one stream are safe.
 */
#define MAMBA_SCAN_NOALLOC_SCRATCH_BYTES ((size_t)8 << 20)
int mamba_scan_fwd_noalloc(int32_t batch, int32_t seqlen, int32_t d_inner, int32_t d_state,
                           int32_t d_conv, int32_t io_dtype, const void* x, const void* dt, const void* z,
                           const void* B, const void* C, const float* conv_w, const float* conv_b,
                           const float* dt_bias, const float* D, const float* A,
                           const float* conv_state_in, const float* ssm_state_in, void* y,
                           float* conv_state_out, float* ssm_state_out, void* stream);

/* Bytes of the checkpoint array of mamba_scan_fwd_ckpt / mamba_scan_bwd_ckpt:
   [batch][ceil(seqlen / 16)][d_inner][16] float32 (0 for shapes they reject:
   d_state other than 16, d_inner > 2^24). */
size_t mamba_scan_ckpt_bytes(int32_t batch, int32_t seqlen, int32_t d_inner, int32_t d_state);

/*
 * Training prefill: mamba_scan_fwd (same arguments, outputs, workspace,
 * validation and errors) that also writes
 *
 *   ckpt            [batch][ceil(seqlen / 16)][d_inner][16] float32, 4-byte
 *                   aligned, mamba_scan_ckpt_bytes(...) bytes; entry [b][s][d][n]
 *                   is state n of channel d before timestep 16 s (the state of
 *                   the recurrence of calm-mamba 0.1.4 PKG-INFO, "Mamba
 *                   operator", step 5; ssm_state_in, or zeros, for s = 0).
 *
 * These are the states mamba_scan_bwd recomputes before its adjoint pass;
 * handing them to mamba_scan_bwd_ckpt skips that pass. d_state must be 16;
 * ckpt must not overlap any input or output. With an unsplit sequence (the
 * usual case at training shapes) the values equal mamba_scan_bwd's own
 * recomputation bit for bit.
 */
int mamba_scan_fwd_ckpt(int32_t batch, int32_t seqlen, int32_t d_inner, int32_t d_state,
                        int32_t d_conv, int32_t io_dtype, const void* x, const void* dt, const void* z,
                        const void* B, const void* C, const float* conv_w, const float* conv_b,
                        const float* dt_bias, const float* D, const float* A,
                        const float* conv_state_in, const float* ssm_state_in, void* y,
                        float* conv_state_out, float* ssm_state_out, float* ckpt, void* workspace,
                        size_t workspace_bytes, void* stream);

/* Bytes of device workspace mamba_scan_bwd needs (0 for shapes it rejects). */
size_t mamba_scan_bwd_workspace_bytes(int32_t batch, int32_t seqlen, int32_t d_inner, int32_t d_state,
                                      int32_t io_dtype);

/*
 * Backward of mamba_scan_fwd (calm-mamba 0.1.4 PKG-INFO, "GPU acceleration":
 * the backward recomputes the forward): given dy = dL/dy, the gradients of L
 * with respect to the inputs and parameters of the same call.
 *
 *   inputs          x, dt, z, B, C, conv_w, conv_b, dt_bias, D, A,
 *                   conv_state_in, ssm_state_in: as mamba_scan_fwd (states may
 *                   be NULL = zeros; they enter the forward but get no gradient)
 *   dy              [batch][seqlen][d_inner]  io
 *   dx, ddt, dz     [batch][seqlen][d_inner]  io   (outputs)
 *   dB, dC          [batch][seqlen][d_state]  f32  (outputs; summed over channels)
 *   dconv_w [d_inner][d_conv], dconv_b, ddt_bias, dD [d_inner], dA [d_inner][d_state]
 *                   f32 outputs, summed over batch rows and timesteps
 *   workspace       >= mamba_scan_bwd_workspace_bytes(...) bytes, 16-byte
 *                   aligned (checkpoints of the state every 16 steps and
 *                   per-workgroup partial sums)
 * d_state must be 16, d_inner <= 2^24, batch * ceil(d_inner / 16) < 2^24 and
 * batch * seqlen < 2^28 (the kernels' grids count work-items in 32 bits);
 * other shapes are MAMBA_ERR_SHAPE. Every output is overwritten (none
 * accumulates); outputs may not overlap inputs or one another. Sums are taken
 * in a fixed order, so results are deterministic. Same conventions and errors
 * as mamba_scan_fwd.
 */
int mamba_scan_bwd(int32_t batch, int32_t seqlen, int32_t d_inner, int32_t d_state, int32_t d_conv,
                   int32_t io_dtype, const void* x, const void* dt, const void* z, const void* B, const void* C,
                   const float* conv_w, const float* conv_b, const float* dt_bias, const float* D, const float* A,
                   const float* conv_state_in, const float* ssm_state_in, const void* dy, void* dx, void* ddt,
                   void* dz, float* dB, float* dC, float* dconv_w, float* dconv_b, float* ddt_bias, float* dD,
                   float* dA, void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of device workspace mamba_scan_bwd_ckpt needs (0 for shapes it
   rejects): that of mamba_scan_bwd less the checkpoints. */
size_t mamba_scan_bwd_ckpt_workspace_bytes(int32_t batch, int32_t seqlen, int32_t d_inner, int32_t d_state,
                                           int32_t io_dtype);

/*
 * mamba_scan_bwd from the checkpoints that mamba_scan_fwd_ckpt wrote for the
 * same inputs (ckpt: an input, as described there), so that the backward's
 * own forward pass is skipped. Same arguments, outputs, validation and errors
 * as mamba_scan_bwd otherwise; workspace >=
 * mamba_scan_bwd_ckpt_workspace_bytes(...) bytes, 16-byte aligned. Given the
 * checkpoints of mamba_scan_fwd_ckpt's unsplit path the results equal
 * mamba_scan_bwd's bit for bit.
 */
int mamba_scan_bwd_ckpt(int32_t batch, int32_t seqlen, int32_t d_inner, int32_t d_state, int32_t d_conv,
                        int32_t io_dtype, const void* x, const void* dt, const void* z, const void* B, const void* C,
                        const float* conv_w, const float* conv_b, const float* dt_bias, const float* D,
                        const float* A, const float* conv_state_in, const float* ssm_state_in, const void* dy,
                        void* dx, void* ddt, void* dz, float* dB, float* dC, float* dconv_w, float* dconv_b,
                        float* ddt_bias, float* dD, float* dA, const float* ckpt, void* workspace,
                        size_t workspace_bytes, void* stream);

/*
 * One decode step: one token per batch row (niverel-mamba 0.1.0 PKG-INFO,
 * "Autoregressive decoding"; calm-mamba 0.1.4 PKG-INFO, O(1) state-cached
 * generation). Same arithmetic as mamba_scan_fwd with seqlen = 1; the conv
 * window is (conv_state_in[0..d_conv-2], x) and the new conv state drops the
 * oldest entry and appends x.
 *
 *   x, dt, z        [batch][d_inner]          io
 *   B, C            [batch][d_state]          io
 *   conv_w, conv_b, dt_bias, D, A             f32, as for mamba_scan_fwd
 *   conv_state_in   [batch][d_inner][d_conv-1] f32, required
 *   ssm_state_in    [batch][d_inner][d_state]  f32, required
 *   y               [batch][d_inner]          io   (output; must not overlap any input)
 *   conv_state_out, ssm_state_out             f32, required; each may be exactly
 *                   its input (in place) or disjoint from every input.
 * batch*d_inner < 2^31; the states themselves may hold more elements than
 * that (tested at 34.6 GB of ssm state).
 */
int mamba_scan_step(int32_t batch, int32_t d_inner, int32_t d_state, int32_t d_conv,
                    int32_t io_dtype, const void* x, const void* dt, const void* z, const void* B,
                    const void* C, const float* conv_w, const float* conv_b, const float* dt_bias,
                    const float* D, const float* A, const float* conv_state_in,
                    const float* ssm_state_in, void* y, float* conv_state_out,
                    float* ssm_state_out, void* stream);

/*
 * One token from its activated conv output (the decode counterpart of
 * mamba_scan_fwd_xc): xc [batch][d_inner] io replaces x; there are no conv
 * weights and no conv states (the caller keeps the conv history). The B and
 * C rows of batch row b start b * bc_stride elements past their pointers
 * (d_state <= bc_stride <= 2^24; batch * bc_stride < 2^31). dt, z, dt_bias, D, A,
 * ssm_state_in, y and ssm_state_out are as for mamba_scan_step (the SSM state
 * may be updated in place). Same validation and statuses.
 */
int mamba_scan_step_xc(int32_t batch, int32_t d_inner, int32_t d_state, int32_t io_dtype, const void* xc,
                       const void* dt, const void* z, const void* B, const void* C, int32_t bc_stride,
                       const float* dt_bias, const float* D, const float* A, const float* ssm_state_in, void* y,
                       float* ssm_state_out, void* stream);

/*
 * One token from its activated conv output with dt_proj inside (calm-mamba
 * 0.1.4 PKG-INFO, "Mamba operator", step 4's projection and softplus fused
 * with steps 5-6 around the scan, for a decoding layer): as
 * mamba_scan_step_xc, except that dt is not passed; it is computed per
 * (b, d) as
 *   dt[b][d] = sum_k dt_low[b][k] * w_dt[d][k],  k < dt_rank,
 * in float32 and rounded to io_dtype (the value a layer storing dt in that
 * dtype would read back), then softplus(dt + dt_bias) as usual.
 *
 *   dt_low   rows of dt_rank io elements, row b starting b * dtl_stride
 *            elements past the pointer (x_proj's output read in place)
 *   w_dt     [d_inner][dt_rank] io (dt_proj's weight, torch Linear layout)
 *   z        row b of d_inner io elements starting b * z_stride elements past
 *            the pointer (z_stride = d_inner: contiguous; 2 * d_inner: z read
 *            in place from in_proj's output row x, z); d_inner <= z_stride <= 2^24
 *   1 <= dt_rank <= 4096, dt_rank <= dtl_stride <= 2^24, batch * dtl_stride
 *   and batch * z_stride below 2^31.
 * The other arguments, validation (dt_low and w_dt count as inputs in the
 * aliasing rules, z covers the elements from its first to the end of its
 * last row) and statuses are those of mamba_scan_step_xc.
 */
int mamba_scan_step_xc_dtproj(int32_t batch, int32_t d_inner, int32_t d_state, int32_t dt_rank,
                              int32_t io_dtype, const void* xc, const void* dt_low, int32_t dtl_stride,
                              const void* w_dt, const void* z, int32_t z_stride, const void* B, const void* C,
                              int32_t bc_stride, const float* dt_bias, const float* D, const float* A,
                              const float* ssm_state_in, void* y, float* ssm_state_out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MAMBA_SCAN_H */
