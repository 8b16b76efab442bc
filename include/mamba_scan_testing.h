/*
 * mamba_scan_testing.h — testing entry points of libmamba_scan.
 *
 * For test suites only (the product entry points of include/mamba_scan.h plan
 * every call as a pure function of its shape and never consult these). They
 * let a test run every prefill kernel family on any shape, so that each
 * family's split and unsplit paths, and the row kernel's per-stage-descriptor
 * path, are checked against a reference without building the library twice.
 * The computation is the one mamba_scan_fwd / mamba_scan_fwd_seq /
 * mamba_scan_fwd_ckpt define (calm-mamba 0.1.4 PKG-INFO, "Architecture",
 * "Mamba operator", steps 2, 4, 5 and 6; packed documents: niverel-mamba
 * 0.1.0 PKG-INFO, "seq_idx strict reset"); only the choice of kernels
 * differs, so results agree with the product call up to floating-point
 * rounding (bit for bit when the same kernel family and split are taken).
 */
#ifndef MAMBA_SCAN_TESTING_H
#define MAMBA_SCAN_TESTING_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Workspace (bytes) that mamba_scan_testing_fwd needs for `kind` (see below)
 * and this shape, with or without checkpoints or document ids; 0 for an
 * invalid kind or shape (same shape rules as mamba_scan_fwd). */
size_t mamba_scan_testing_fwd_workspace_bytes(int32_t kind, int32_t batch, int32_t seqlen, int32_t d_inner,
                                              int32_t d_state, int32_t io_dtype);

/* The prefill of mamba_scan_fwd with the kernel family chosen by the caller.
 *   kind       -1 = the product plan; 0 = one lane per channel; 1 = four lanes
 *              per channel; 2 = sixteen lanes per channel (d_state 16 only;
 *              for d_state 8 the product plan is used). The sequence split
 *              is planned for the chosen family as usual.
 *   force_wide non-zero: the sixteen-lane kernel builds its buffer
 *              descriptors at every stage (the path it takes by itself when a
 *              chunk spans 2 GiB or more); results are bit-identical.
 *   seq_idx    NULL, or document ids as for mamba_scan_fwd_seq (not with kind 0).
 *   ckpt       NULL, or the checkpoints of mamba_scan_fwd_ckpt (kind -1 or 2,
 *              no seq_idx).
 * Every other argument, layout, ownership rule and status is that of
 * mamba_scan_fwd (include/mamba_scan.h); an invalid kind, or checkpoints
 * combined with seq_idx or another family, returns MAMBA_ERR_SHAPE before any
 * HIP call. Successful calls are counted like the product calls. */
int mamba_scan_testing_fwd(int32_t kind, int32_t force_wide, int32_t batch, int32_t seqlen, int32_t d_inner,
                           int32_t d_state, int32_t d_conv, int32_t io_dtype, const void* x, const void* dt,
                           const void* z, const void* B, const void* C, const int32_t* seq_idx,
                           const float* conv_w, const float* conv_b, const float* dt_bias, const float* D,
                           const float* A, const float* conv_state_in, const float* ssm_state_in, void* y,
                           float* conv_state_out, float* ssm_state_out, float* ckpt, void* workspace,
                           size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MAMBA_SCAN_TESTING_H */
