// Host-side interface between the C-ABI layer (mamba_scan_api.cpp) and the
// kernel launchers (scan_fwd.hip, scan_step.hip). Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace mscan {

// Validated arguments of one prefill call (see mamba_scan_fwd in
// include/mamba_scan.h for meaning and layout).
struct FwdCall {
  int32_t batch, seqlen, d_inner, d_state, io_dtype;
  const void *x, *dt, *z, *B, *C;
  const int32_t* seq_idx;  // [batch][seqlen] document ids, or NULL (no resets)
  const float *conv_w, *conv_b, *dt_bias, *D, *A;
  const float *conv_state_in, *ssm_state_in;
  void* y;
  float *conv_state_out, *ssm_state_out;
  float* workspace;
  hipStream_t stream;
  float* ckpt = nullptr;  // [batch][ceil(seqlen/16)][d_inner][16]: states before each 16-step stage, or NULL
  bool force_wide = false;  // row kernel: per-stage buffer descriptors at any size (testing entry point only)
  bool xc_input = false;    // x holds the activated conv output xc: no conv, SiLU or conv state (no seq_idx, no ckpt)
  int32_t bc_stride = 0;    // elements between consecutive rows of B and of C (>= d_state)
  // dt_proj inside the prefill (xc input, row kernel only): when dt_low is
  // set, dt[b][t][d] is dt_low[b][t] . w_dt[d] over dt_rank terms (a multiple
  // of 8, at most 64) on the matrix cores, and the dt pointer is unused
  const void* dt_low = nullptr;
  int32_t dtl_stride = 0;
  const void* w_dt = nullptr;
  int32_t dt_rank = 0;
  int32_t z_stride = 0;  // with dt_low: elements between consecutive rows (b, t) of z (0 = d_inner)
  // row kernel, with ckpt and a one-chunk plan (chunk_len = seqlen): the
  // checkpoints only (no y, states or summaries; z, C, D and y may be NULL)
  bool ckpt_only = false;
};

struct StepCall {
  int32_t batch, d_inner, d_state, io_dtype;
  const void *x, *dt, *z, *B, *C;
  const float *conv_w, *conv_b, *dt_bias, *D, *A;
  const float *conv_state_in, *ssm_state_in;
  void* y;
  float *conv_state_out, *ssm_state_out;
  hipStream_t stream;
  bool xc_input = false;  // x holds the token's activated conv output: no conv, conv states untouched
  int32_t bc_stride = 0;  // elements between the batch rows of B and of C (>= d_state)
  // dt_proj inside the step (xc input only): when dt_low is set, dt is
  // dt_low[b] . w_dt[d] over dt_rank terms, and the dt pointer is unused
  const void* dt_low = nullptr;
  int32_t dtl_stride = 0;
  const void* w_dt = nullptr;
  int32_t dt_rank = 0;
  int32_t z_stride = 0;  // with dt_low: elements between the batch rows of z (0 = d_inner)
};

// How a prefill call is run: which kernel family, and how the sequence is
// split into chunks.
enum FwdKind { kFwdChannel = 0, kFwdQuad = 1, kFwdRow = 2 };
struct FwdPlan {
  int32_t kind;       // FwdKind
  int32_t n_chunks;   // number of sequence chunks (1 = no split)
  int32_t chunk_len;  // timesteps per chunk (last chunk may be shorter)
  size_t ws_floats;   // float32 workspace elements needed
};

// Workspace of the four-lanes-per-channel prefill (float32 offsets; all zero
// when the sequence is not split).
struct QuadWs {
  size_t sum_S, sum_delta, sum_reset, ssm_copy, conv_copy, total;
};
QuadWs quad_ws_layout(int32_t batch, int32_t d_inner, int32_t d_state, int32_t n_chunks);
hipError_t launch_fwd_quad(const FwdCall& c, const FwdPlan& p);
hipError_t launch_fwd_row(const FwdCall& c, const FwdPlan& p);  // d_state 16 only

// Validated arguments of one backward call (see mamba_scan_bwd in
// include/mamba_scan.h).
struct BwdCall {
  int32_t batch, seqlen, d_inner, d_state, io_dtype;
  const void *x, *dt, *z, *B, *C;
  const float *conv_w, *conv_b, *dt_bias, *D, *A;
  const float *conv_state_in, *ssm_state_in;
  const void* dy;
  void *dx, *ddt, *dz;
  float *dB, *dC, *dconv_w, *dconv_b, *ddt_bias, *dD, *dA;
  float* workspace;
  hipStream_t stream;
  const float* ckpt = nullptr;  // checkpoints from the forward; NULL: the backward computes them in its workspace
};
// Workspace of the backward (float32 offsets); without own_ckpt the
// checkpoints come from the caller and take no workspace.
struct BwdWs {
  size_t ckpt, dBpart, dCpart, pgrad, total;
};
BwdWs bwd_ws_layout(int32_t batch, int32_t seqlen, int32_t d_inner, bool own_ckpt = true);
size_t ckpt_floats(int32_t batch, int32_t seqlen, int32_t d_inner);  // d_state 16
hipError_t launch_bwd(const BwdCall& c);  // d_state 16

// Mamba-2 SSD scan (headdim 64, d_state 64 or 128).
struct SsdCall {
  int32_t batch, seqlen, nheads, headdim, d_state, ngroups, io_dtype;
  const void *x, *dt, *B, *C;
  const int32_t* seq_idx;  // NULL: one document per row
  const float *dt_bias, *A, *D, *state_in;
  void* y;
  float* state_out;
  float* workspace;
  hipStream_t stream;
};
// Workspace of the SSD scan (float32 offsets): per (batch, chunk, head) state
// [64][d_state], chunk decay, and the chunk's cumulative log-decay, delta and
// latest document start at or before each step ([256] each).
struct SsdWs {
  size_t states, decay, cs, dl, sg, total;
};
SsdWs ssd_ws_layout(int32_t batch, int32_t seqlen, int32_t nheads, int32_t d_state);
hipError_t launch_ssd(const SsdCall& c);
hipError_t launch_ssd_step(const SsdCall& c);  // one token: seqlen unused, workspace unused

// The plan of a prefill call: a pure function of the shape. `forced_kind` >= 0
// (a FwdKind; testing entry point only) takes that kernel family instead of
// the planned one, with the sequence split planned for it as usual.
FwdPlan plan_fwd(int32_t batch, int32_t seqlen, int32_t d_inner, int32_t d_state, int32_t io_dtype,
                 int32_t forced_kind = -1);
// The plan of a prefill that also writes checkpoints: the sixteen-lane row
// kernel (d_state 16), with the sequence split as plan_fwd would split it.
FwdPlan plan_fwd_row(int32_t batch, int32_t seqlen, int32_t d_inner, int32_t io_dtype);

// The fixed device scratch of mamba_scan_fwd_noalloc: its size, and its
// address on device `dev` (the current device; looked up once per device).
size_t noalloc_scratch_bytes();
hipError_t noalloc_scratch(int dev, void** ptr);

// Enqueue the kernels; return the first HIP error (hipSuccess if none).
hipError_t launch_fwd(const FwdCall& c, const FwdPlan& p);
hipError_t launch_step(const StepCall& c);

}  // namespace mscan
