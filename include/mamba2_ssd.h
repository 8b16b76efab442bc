/*
 * mamba2_ssd.h -- C ABI of the Mamba-2 SSD scan in libmamba_scan.so (MI355X,
 * gfx950). Status codes, threading, stream and error conventions are those of
 * mamba_scan.h (validation before any HIP call, MAMBA_ERR_* codes, the
 * thread's detail in mamba_scan_last_error(), no fallback of any kind).
 *
 * The operation (niverel-mamba 0.1.0 PKG-INFO, "The weight contract": heads of
 * headdim 64 with one dt_bias, A_log and D each, B and C shared by the heads of
 * a group; "What is *not* promised": chunked evaluation with the decay
 * exp(cs_l - cs_s) over a chunk-wide cumulative sum), per batch row b and head
 * h of group g = h / (nheads / ngroups), with a state matrix
 * S[headdim][d_state]:
 *
 *   delta_t = softplus(dt[b,t,h] + dt_bias[h])
 *   S       = exp(delta_t * A[h]) * S + delta_t * x[b,t,h,:] (outer) B[b,t,g,:]
 *   y[b,t,h,:] = S C[b,t,g,:] + D[h] * x[b,t,h,:]
 *
 * evaluated in chunks of 256 steps on the matrix cores (float32 accumulation;
 * bfloat16 io uses bfloat16 operands, float32 io float32 operands). The result
 * equals the sequential recurrence up to rounding; it is not bitwise equal to
 * it, but it is bitwise reproducible run to run.
 */
#ifndef MAMBA2_SSD_H
#define MAMBA2_SSD_H

#include <stddef.h>
#include <stdint.h>

#include "mamba_scan.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Bytes of device workspace mamba2_ssd_fwd needs (0 for shapes it rejects):
   one float32 [headdim][d_state] state and one decay per (batch row, chunk of
   256 steps, head). */
size_t mamba2_ssd_fwd_workspace_bytes(int32_t batch, int32_t seqlen, int32_t nheads, int32_t headdim,
                                      int32_t d_state, int32_t ngroups, int32_t io_dtype);

/*
 * Whole-sequence SSD scan. All pointers are device pointers owned by the caller.
 *   x            [batch][seqlen][nheads][headdim]  io, 16-byte aligned
 *   dt           [batch][seqlen][nheads]           io (before dt_bias and softplus)
 *   B, C         [batch][seqlen][ngroups][d_state] io, 16-byte aligned
 *   dt_bias, A, D  [nheads] float32 (A = -exp(A_log), given)
 *   state_in     [batch][nheads][headdim][d_state] float32, 16-byte aligned, or NULL (zeros)
 *   y            [batch][seqlen][nheads][headdim]  io, 16-byte aligned (must not overlap any input)
 *   state_out    like state_in, or NULL (not written); may be exactly state_in
 *   workspace    >= mamba2_ssd_fwd_workspace_bytes(...) bytes, 256-byte aligned
 * headdim must be 64, d_state 64 or 128, ngroups >= 1 dividing nheads;
 * batch and nheads <= 65535; batch*seqlen*nheads*headdim < 2^31.
 * Returns MAMBA_OK or a MAMBA_ERR_* status; asynchronous on `stream`.
 */
int mamba2_ssd_fwd(int32_t batch, int32_t seqlen, int32_t nheads, int32_t headdim, int32_t d_state, int32_t ngroups,
                   int32_t io_dtype, const void* x, const void* dt, const void* B, const void* C,
                   const float* dt_bias, const float* A, const float* D, const float* state_in, void* y,
                   float* state_out, void* workspace, size_t workspace_bytes, void* stream);

/*
 * mamba2_ssd_fwd over packed documents (niverel-mamba 0.1.0 PKG-INFO, "seq_idx
 * strict reset"): seq_idx [batch][seqlen] int32 document ids (4-byte aligned,
 * required, an input); the state restarts from zero before every step whose id
 * differs from the previous step's, wherever that falls in a chunk. state_in
 * seeds the first document of each row; state_out is the state after the last
 * step. A constant seq_idx gives exactly the result of mamba2_ssd_fwd.
 */
int mamba2_ssd_fwd_seq(int32_t batch, int32_t seqlen, int32_t nheads, int32_t headdim, int32_t d_state,
                       int32_t ngroups, int32_t io_dtype, const void* x, const void* dt, const void* B,
                       const void* C, const int32_t* seq_idx, const float* dt_bias, const float* A, const float* D,
                       const float* state_in, void* y, float* state_out, void* workspace, size_t workspace_bytes,
                       void* stream);

/*
 * One token per batch row (niverel-mamba 0.1.0 PKG-INFO, "Autoregressive
 * decoding": the step is functional in the state), the same recurrence as
 * mamba2_ssd_fwd for seqlen 1.
 *   x            [batch][nheads][headdim]       io
 *   dt           [batch][nheads]                io
 *   B, C         [batch][ngroups][d_state]      io
 *   dt_bias, A, D  [nheads] float32
 *   state_in     [batch][nheads][headdim][d_state] float32, 16-byte aligned, required
 *   y            [batch][nheads][headdim]       io (must not overlap any input)
 *   state_out    like state_in, required; may be exactly state_in (in place)
 * Same shape limits as mamba2_ssd_fwd (batch*nheads*headdim < 2^31); the state
 * itself may hold more elements than that (tested at 34.6 GB). No workspace.
 */
int mamba2_ssd_step(int32_t batch, int32_t nheads, int32_t headdim, int32_t d_state, int32_t ngroups,
                    int32_t io_dtype, const void* x, const void* dt, const void* B, const void* C,
                    const float* dt_bias, const float* A, const float* D, const float* state_in, void* y,
                    float* state_out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MAMBA2_SSD_H */
