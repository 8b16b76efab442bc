// Host-side interface between the mixer's C ABI (mamba_mixer.cpp) and its
// kernels (mixer_conv.hip). Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mmix {

// x is read from rows xs elements apart (d_inner, or 2 * d_inner in
// in_proj's output rows x, z); xc is written contiguous.
// xc[b][t][d] = SiLU(conv(x)) for the whole sequence; conv0 may be NULL (zeros).
hipError_t launch_conv_silu(int io_dtype, int32_t batch, int32_t seqlen, int32_t d_inner, const void* x, int32_t xs,
                            const float* conv_w, const float* conv_b, const float* conv0, void* xc,
                            hipStream_t stream);
// The conv state after the last token: cso[b][d][j] = element seqlen-3+j of
// (conv0 ++ x) (conv0 may be NULL: zeros; cso may equal conv0).
hipError_t launch_conv_state(int io_dtype, int32_t batch, int32_t seqlen, int32_t d_inner, const void* x, int32_t xs,
                             const float* conv0, float* cso, hipStream_t stream);
// One token: xc[b][d] from conv_state[b][d][0..2] and x[b][d], and the new
// conv state (conv_state[1], conv_state[2], x) into conv_state_out (which may
// be conv_state).
hipError_t launch_conv_silu_step(int io_dtype, int32_t batch, int32_t d_inner, const void* x, int32_t xs,
                                 const float* conv_w, const float* conv_b, const float* conv_state, void* xc,
                                 float* conv_state_out, hipStream_t stream);

}  // namespace mmix
