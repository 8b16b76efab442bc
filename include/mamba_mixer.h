/*
 * mamba_mixer.h -- C ABI of libmamba_mixer.so: one whole Mamba-1 mixer layer
 * on MI355X (gfx950), built around the selective scan of libmamba_scan.so.
 *
 * The layer (calm-mamba 0.1.4 PKG-INFO, "Architecture" / "Mamba operator",
 * steps 1-7), for hidden states u [tokens][d_model]:
 *
 *   1  x  = u W_in[0:D]^T,  z = u W_in[D:2D]^T          (in_proj, no bias)
 *   2  xc = SiLU(causal depthwise conv1d(x) + conv_b)    (kernel 4)
 *   3  dt_low = xc W_x[0:R]^T, B = xc W_x[R:R+N]^T,
 *      C = xc W_x[R+N:R+2N]^T                            (x_proj, no bias)
 *   4  dt = dt_low W_dt^T; delta = softplus(dt + dt_bias) (dt_proj + softplus)
 *   5  h = exp(delta A) h + delta B xc;  y = C.h + D xc  (selective scan)
 *   6  y = y * SiLU(z)                                   (gate)
 *   7  out = y W_out^T                                   (out_proj, no bias)
 *
 * with D = d_inner, N = d_state, R = dt_rank. Step 2 runs in a kernel of this
 * library, which also writes the new conv state; its output xc feeds x_proj
 * and the scan (mamba_scan_fwd_xc / mamba_scan_step_xc run steps 4-6 from it
 * without a second conv). The projections are plain GEMMs, run with rocBLAS
 * (bf16 or fp32 inputs, fp32 accumulation): in_proj (for a sequence as its x
 * and z halves into contiguous arrays; for one token as one GEMM whose output
 * row holds the token's x and then its z, which the conv and the scan step
 * read there with a row stride of 2 * d_inner), x_proj as one GEMM whose
 * output row holds the token's dt_low, B and C side by side (the scan reads
 * them there), out_proj. dt_proj runs inside the
 * scan: on the matrix cores in the prefill (mamba_scan_fwd_xc_dtproj, for
 * d_state 16 and dt_rank a multiple of 8 up to 64; other shapes take a
 * dt_proj GEMM and mamba_scan_fwd_xc) and in the one-token step
 * (mamba_scan_step_xc_dtproj); either way dt is rounded to the io dtype, the
 * value a stored dt would hold.
 *
 * Conventions are those of mamba_scan.h (device pointers owned by the caller,
 * asynchronous on `stream`, validation before any launch, status codes of
 * mamba_status, no fallback), with these additions:
 *  - Weight matrices use the torch Linear layout [out_features][in_features]
 *    in the io dtype; conv_w [d_inner][4], conv_b, dt_bias, D [d_inner] and
 *    A [d_inner][d_state] are float32, as in mamba_scan.h.
 *  - Every intermediate (x, z, xc, dt_low, B, C, dt, y) is stored in the io
 *    dtype in the caller's workspace, so bfloat16 layers round them there,
 *    and the later steps consume the stored values (the scan reads the
 *    stored xc). The pages give the steps but not the layer's storage
 *    precision; this is the reading taken (a Mamba layer in bfloat16 keeps
 *    its activations in bfloat16 between kernels).
 *  - The library holds one rocBLAS handle per thread and device (created on
 *    first use; rocBLAS keeps its own device workspace).
 */
#ifndef MAMBA_MIXER_H
#define MAMBA_MIXER_H

#include <stddef.h>
#include <stdint.h>

#include "mamba_scan.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Human-readable detail of this thread's last failed mixer call ("" if none).
   Owned by the library, valid until the thread's next mixer call. */
const char* mamba_mixer_last_error(void);

/* Bytes of device workspace mamba_mixer_fwd needs (a pure function of the
   arguments, 0 for shapes mamba_mixer_fwd would reject). */
size_t mamba_mixer_fwd_workspace_bytes(int32_t batch, int32_t seqlen, int32_t d_model, int32_t d_inner,
                                       int32_t d_state, int32_t dt_rank, int32_t io_dtype);

/*
 * Whole-sequence mixer layer.
 *   hidden          [batch][seqlen][d_model]        io
 *   w_in            [2*d_inner][d_model]            io  (rows 0..d_inner-1 give x, the rest z)
 *   conv_w, conv_b  as mamba_scan_fwd               f32
 *   w_x             [dt_rank + 2*d_state][d_inner]  io  (rows give dt_low, then B, then C)
 *   w_dt            [d_inner][dt_rank]              io
 *   dt_bias, A, D   as mamba_scan_fwd               f32
 *   w_out           [d_model][d_inner]              io
 *   conv_state_in, ssm_state_in, conv_state_out, ssm_state_out: as mamba_scan_fwd
 *   out             [batch][seqlen][d_model]        io  (must not overlap any input)
 *   workspace       >= mamba_mixer_fwd_workspace_bytes(...) bytes, 256-byte aligned
 * d_conv must be 4, d_state 8 or 16, dt_rank >= 1; batch*seqlen*max(2*d_inner,
 * d_model) < 2^31.
 */
int mamba_mixer_fwd(int32_t batch, int32_t seqlen, int32_t d_model, int32_t d_inner, int32_t d_state,
                    int32_t dt_rank, int32_t d_conv, int32_t io_dtype, const void* hidden, const void* w_in,
                    const float* conv_w, const float* conv_b, const void* w_x, const void* w_dt,
                    const float* dt_bias, const float* A, const float* D, const void* w_out,
                    const float* conv_state_in, const float* ssm_state_in, void* out, float* conv_state_out,
                    float* ssm_state_out, void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of device workspace mamba_mixer_step needs. */
size_t mamba_mixer_step_workspace_bytes(int32_t batch, int32_t d_model, int32_t d_inner, int32_t d_state,
                                        int32_t dt_rank, int32_t io_dtype);

/*
 * One token per batch row through the layer (niverel-mamba 0.1.0 PKG-INFO,
 * "Autoregressive decoding": functional in the states).
 *   hidden          [batch][d_model]                io
 *   weights         as mamba_mixer_fwd
 *   conv_state_in, ssm_state_in, conv_state_out, ssm_state_out: required, as
 *                   mamba_scan_step (each output may be exactly its input)
 *   out             [batch][d_model]                io
 *   workspace       >= mamba_mixer_step_workspace_bytes(...) bytes, 256-byte aligned
 */
int mamba_mixer_step(int32_t batch, int32_t d_model, int32_t d_inner, int32_t d_state, int32_t dt_rank,
                     int32_t d_conv, int32_t io_dtype, const void* hidden, const void* w_in, const float* conv_w,
                     const float* conv_b, const void* w_x, const void* w_dt, const float* dt_bias, const float* A,
                     const float* D, const void* w_out, const float* conv_state_in, const float* ssm_state_in,
                     void* out, float* conv_state_out, float* ssm_state_out, void* workspace,
                     size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MAMBA_MIXER_H */
