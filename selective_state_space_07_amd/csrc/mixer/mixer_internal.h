// Host-side interface between the mixer's C ABI (mamba_mixer.cpp) and its
// kernels (mixer_conv.hip). Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mmix {

// xc[b][t][d] = SiLU(conv(x)) for the whole sequence; conv0 may be NULL (zeros).
hipError_t launch_conv_silu(int io_dtype, int32_t batch, int32_t seqlen, int32_t d_inner, const void* x,
                            const float* conv_w, const float* conv_b, const float* conv0, void* xc,
                            hipStream_t stream);
// One token: xc[b][d] from conv_state[b][d][0..2] and x[b][d].
hipError_t launch_conv_silu_step(int io_dtype, int32_t batch, int32_t d_inner, const void* x, const float* conv_w,
                                 const float* conv_b, const float* conv_state, void* xc, hipStream_t stream);

}  // namespace mmix
