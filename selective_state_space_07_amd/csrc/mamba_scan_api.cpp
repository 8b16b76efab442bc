// C-ABI layer of libmamba_scan: argument validation, planning, device check
// and the call counter. Every check runs before any HIP call, so invalid
// arguments never reach the device (declared in include/mamba_scan.h).
#include "../../include/mamba_scan.h"
#include "../../include/mamba2_ssd.h"
#include "../../include/mamba_scan_testing.h"

#include <hip/hip_runtime.h>

#include <atomic>
#include <initializer_list>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>

#include "scan_internal.h"

namespace {

thread_local std::string g_last_error;
std::atomic<uint64_t> g_calls{0};

int fail(int status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = std::string(mamba_scan_status_str(status)) + ": " + buf;
  return status;
}

int ok() {
  g_last_error.clear();
  return MAMBA_OK;
}

size_t io_size(int32_t io_dtype) { return io_dtype == MAMBA_BF16 ? 2 : 4; }

struct Range {
  const char* name;
  uintptr_t lo, hi;  // [lo, hi)
};

Range range(const char* name, const void* p, size_t bytes) {
  const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
  return Range{name, lo, p ? lo + bytes : lo};
}

bool overlaps(const Range& a, const Range& b) {
  return a.lo != 0 && b.lo != 0 && a.lo < b.hi && b.lo < a.hi;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Whether the product of non-negative 32-bit extents stays below 2^31,
// evaluated without overflow (each partial product is checked before the
// next factor, so it never exceeds 2^62).
bool below_2_31(std::initializer_list<int64_t> factors) {
  int64_t p = 1;
  for (const int64_t f : factors) {
    if (f < 0) return false;
    p *= f;
    if (p >= (int64_t{1} << 31)) return false;
  }
  return true;
}

int check_dims(int32_t batch, int32_t seqlen, int32_t d_inner, int32_t d_state, int32_t d_conv) {
  if (batch < 1 || seqlen < 1 || d_inner < 1 || d_state < 1)
    return fail(MAMBA_ERR_SHAPE, "dims must be >= 1 (batch=%d seqlen=%d d_inner=%d d_state=%d)", batch,
                seqlen, d_inner, d_state);
  if (d_conv != 4) return fail(MAMBA_ERR_SHAPE, "d_conv must be 4 (got %d)", d_conv);
  if (d_state != 8 && d_state != 16) return fail(MAMBA_ERR_SHAPE, "d_state must be 8 or 16 (got %d)", d_state);
  const int64_t widest = d_inner > d_state ? d_inner : d_state;
  if (!below_2_31({batch, seqlen, widest}) || !below_2_31({d_inner, d_state}))
    return fail(MAMBA_ERR_SHAPE, "tensor too large (batch*seqlen*max(d_inner,d_state) must be < 2^31)");
  return MAMBA_OK;
}

// Outputs may not overlap inputs, except that a state output may coincide
// exactly with its own state input. Outputs may not overlap one another.
int check_alias(const Range* ins, int n_in, const Range* outs, int n_out, const Range* pair_in,
                const Range* pair_out, int n_pairs) {
  for (int o = 0; o < n_out; ++o) {
    for (int i = 0; i < n_in; ++i) {
      if (!overlaps(outs[o], ins[i])) continue;
      bool exact_pair = false;
      for (int p = 0; p < n_pairs; ++p) {
        if (std::strcmp(outs[o].name, pair_out[p].name) == 0 && std::strcmp(ins[i].name, pair_in[p].name) == 0 &&
            outs[o].lo == ins[i].lo && outs[o].hi == ins[i].hi)
          exact_pair = true;
      }
      if (!exact_pair)
        return fail(MAMBA_ERR_ALIAS, "output %s overlaps input %s (only an exact in-place state update is allowed)",
                    outs[o].name, ins[i].name);
    }
    for (int o2 = o + 1; o2 < n_out; ++o2)
      if (overlaps(outs[o], outs[o2]))
        return fail(MAMBA_ERR_ALIAS, "outputs %s and %s overlap", outs[o].name, outs[o2].name);
  }
  return MAMBA_OK;
}

int check_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
    (void)hipGetLastError();
    return fail(MAMBA_ERR_DEVICE, "no HIP device is visible");
  }
  static std::atomic<int> verified[64];  // 0 = unknown, 1 = gfx950, 2 = other
  const int slot = dev < 64 ? dev : 63;
  int v = verified[slot].load();
  if (v == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
      (void)hipGetLastError();
      return fail(MAMBA_ERR_DEVICE, "hipGetDeviceProperties failed for device %d", dev);
    }
    v = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
    verified[slot].store(v);
    if (v == 2) return fail(MAMBA_ERR_DEVICE, "device %d is %s; this library is built for gfx950 only", dev, prop.gcnArchName);
  }
  if (v != 1) return fail(MAMBA_ERR_DEVICE, "current device is not gfx950; this library is built for gfx950 only");
  return MAMBA_OK;
}

}  // namespace

extern "C" {

int mamba_scan_abi_version(void) { return MAMBA_SCAN_ABI_VERSION; }

const char* mamba_scan_status_str(int status) {
  switch (status) {
    case MAMBA_OK: return "MAMBA_OK";
    case MAMBA_ERR_NULL: return "MAMBA_ERR_NULL";
    case MAMBA_ERR_SHAPE: return "MAMBA_ERR_SHAPE";
    case MAMBA_ERR_DTYPE: return "MAMBA_ERR_DTYPE";
    case MAMBA_ERR_ALIGN: return "MAMBA_ERR_ALIGN";
    case MAMBA_ERR_ALIAS: return "MAMBA_ERR_ALIAS";
    case MAMBA_ERR_WORKSPACE: return "MAMBA_ERR_WORKSPACE";
    case MAMBA_ERR_DEVICE: return "MAMBA_ERR_DEVICE";
    default: return "unknown status";
  }
}

const char* mamba_scan_last_error(void) { return g_last_error.c_str(); }

uint64_t mamba_scan_call_count(void) { return g_calls.load(); }

size_t mamba_scan_fwd_workspace_bytes(int32_t batch, int32_t seqlen, int32_t d_inner, int32_t d_state,
                                      int32_t io_dtype) {
  if (batch < 1 || seqlen < 1 || d_inner < 1 || (d_state != 8 && d_state != 16)) return 0;
  if (io_dtype != MAMBA_F32 && io_dtype != MAMBA_BF16) return 0;
  if (d_inner > (1 << 24)) return 0;
  const int64_t widest = d_inner > d_state ? d_inner : d_state;
  if (!below_2_31({batch, seqlen, widest})) return 0;
  const size_t plain = mscan::plan_fwd(batch, seqlen, d_inner, d_state, io_dtype).ws_floats;
  const size_t row = d_state == 16 ? mscan::plan_fwd_row(batch, seqlen, d_inner, io_dtype).ws_floats : 0;
  return (plain > row ? plain : row) * sizeof(float);
}

size_t mamba_scan_ckpt_bytes(int32_t batch, int32_t seqlen, int32_t d_inner, int32_t d_state) {
  if (batch < 1 || seqlen < 1 || d_inner < 1 || d_inner > (1 << 24) || d_state != 16) return 0;
  if (!below_2_31({batch, seqlen, d_inner})) return 0;
  return mscan::ckpt_floats(batch, seqlen, d_inner) * sizeof(float);
}

namespace {

// The prefill kernels address the rows of one stage through 32-bit buffer
// ranges: 19 rows of d_inner io elements must fit below 2^31 bytes. d_inner is
// capped at 2^24 (64 MiB per float32 row), as for the backward.
constexpr int32_t kMaxFwdDInner = 1 << 24;
// The B / C row stride of the xc entry points: a lane's offset into a stage's
// 16 rows, 15 * bc_stride elements, stays well inside 32 bits.
constexpr int32_t kMaxBcStride = 1 << 24;
// dt_proj inside the decode step: the rank of dt_low (a lane's dot product
// runs over it); Mamba's dt_rank is ceil(d_model / 16).
constexpr int32_t kMaxDtRank = 4096;
// dt_proj inside the prefill: two 32-wide k blocks on the matrix cores, whole
// 8-value fragments per lane.
constexpr int32_t kMaxFwdDtRank = 64;

int fwd_common(int32_t batch, int32_t seqlen, int32_t d_inner, int32_t d_state, int32_t d_conv, int32_t io_dtype,
               const void* x, const void* dt, const void* z, const void* B, const void* C, const int32_t* seq_idx,
               bool want_seq, const float* conv_w, const float* conv_b, const float* dt_bias, const float* D,
               const float* A, const float* conv_state_in, const float* ssm_state_in, void* y,
               float* conv_state_out, float* ssm_state_out, float* ckpt, bool want_ckpt, void* workspace,
               size_t workspace_bytes, void* stream, int32_t forced_kind = -1, bool force_wide = false,
               bool noalloc = false, bool xc_input = false, int32_t bc_stride = 0, bool want_dtp = false,
               const void* dt_low = nullptr, int32_t dtl_stride = 0, const void* w_dt = nullptr,
               int32_t dt_rank = 0, int32_t z_stride = 0) {
  int st = check_dims(batch, seqlen, d_inner, d_state, d_conv);
  if (st) return st;
  if (z_stride == 0) z_stride = d_inner;  // contiguous z
  if (z_stride != d_inner) {               // z read from wider rows (with dt_proj inside)
    if (z_stride < d_inner || z_stride > kMaxBcStride)
      return fail(MAMBA_ERR_SHAPE, "z_stride (%d) must lie in [d_inner, 2^24] (d_inner %d)", z_stride, d_inner);
    if (!below_2_31({batch, seqlen, z_stride}))
      return fail(MAMBA_ERR_SHAPE, "batch * seqlen * z_stride must be below 2^31");
  }
  if (want_dtp) {  // dt comes from dt_low and w_dt; dt itself is not read
    if (d_state != 16) return fail(MAMBA_ERR_SHAPE, "dt_proj inside the prefill serves d_state 16 only (got %d)", d_state);
    if (dt_rank < 8 || dt_rank > kMaxFwdDtRank || dt_rank % 8 != 0)
      return fail(MAMBA_ERR_SHAPE, "dt_rank must be a multiple of 8 in [8, %d] (got %d)", kMaxFwdDtRank, dt_rank);
    if (dtl_stride < dt_rank || dtl_stride > kMaxBcStride)
      return fail(MAMBA_ERR_SHAPE, "dtl_stride (%d) must lie in [dt_rank, 2^24] (dt_rank %d)", dtl_stride, dt_rank);
    if (!below_2_31({batch, seqlen, dtl_stride}))
      return fail(MAMBA_ERR_SHAPE, "batch * seqlen * dtl_stride must be below 2^31");
    if (!dt_low) return fail(MAMBA_ERR_NULL, "dt_low is NULL");
    if (!w_dt) return fail(MAMBA_ERR_NULL, "w_dt is NULL");
    if (io_dtype == MAMBA_F32 || io_dtype == MAMBA_BF16) {
      // dt_low is read in 16-byte pieces from 4-byte aligned offsets
      if (!aligned(dt_low, 4) || (static_cast<size_t>(dtl_stride) * io_size(io_dtype)) % 4 != 0)
        return fail(MAMBA_ERR_ALIGN, "dt_low and its row stride must be 4-byte aligned");
      if (!aligned(w_dt, io_size(io_dtype)))
        return fail(MAMBA_ERR_ALIGN, "w_dt must be %zu-byte aligned", io_size(io_dtype));
    }
    dt = dt_low;  // stands in for dt in the checks below
  }
  if (bc_stride == 0) bc_stride = d_state;  // contiguous B / C rows
  if (bc_stride < d_state || bc_stride > kMaxBcStride)
    return fail(MAMBA_ERR_SHAPE, "bc_stride (%d) must lie in [d_state, 2^24] (d_state %d)", bc_stride, d_state);
  if (!below_2_31({batch, seqlen, bc_stride}))
    return fail(MAMBA_ERR_SHAPE, "batch * seqlen * bc_stride must be below 2^31");
  if (d_inner > kMaxFwdDInner)
    return fail(MAMBA_ERR_SHAPE, "the prefill serves d_inner <= 2^24 (got %d)", d_inner);
  if (io_dtype != MAMBA_F32 && io_dtype != MAMBA_BF16)
    return fail(MAMBA_ERR_DTYPE, "io_dtype must be MAMBA_F32 (0) or MAMBA_BF16 (1), got %d", io_dtype);
  if (want_ckpt) {
    if (d_state != 16) return fail(MAMBA_ERR_SHAPE, "checkpoints serve d_state 16 only (got %d)", d_state);
    if (d_inner > (1 << 24)) return fail(MAMBA_ERR_SHAPE, "checkpoints serve d_inner <= 2^24 (got %d)", d_inner);
    if (!ckpt) return fail(MAMBA_ERR_NULL, "ckpt is NULL");
    if (!aligned(ckpt, 4)) return fail(MAMBA_ERR_ALIGN, "ckpt must be 4-byte aligned");
  }
  const struct { const void* p; const char* n; } req[] = {
      {x, xc_input ? "xc" : "x"}, {dt, "dt"}, {z, "z"}, {B, "B"}, {C, "C"},
      {xc_input ? dt : conv_w, "conv_w"}, {xc_input ? dt : conv_b, "conv_b"},  // no conv with an xc input
      {dt_bias, "dt_bias"}, {D, "D"}, {A, "A"}, {y, "y"}};
  for (const auto& r : req)
    if (!r.p) return fail(MAMBA_ERR_NULL, "%s is NULL", r.n);
  if (want_seq && !seq_idx) return fail(MAMBA_ERR_NULL, "seq_idx is NULL");
  if (want_seq && !aligned(seq_idx, 4)) return fail(MAMBA_ERR_ALIGN, "seq_idx must be 4-byte aligned");
  const size_t es = io_size(io_dtype);
  for (const void* p : {x, dt, z, B, C, static_cast<const void*>(y)})
    if (!aligned(p, es)) return fail(MAMBA_ERR_ALIGN, "io pointers must be %zu-byte aligned", es);
  for (const void* p : {static_cast<const void*>(conv_w), static_cast<const void*>(conv_b),
                        static_cast<const void*>(dt_bias), static_cast<const void*>(D), static_cast<const void*>(A),
                        static_cast<const void*>(conv_state_in), static_cast<const void*>(ssm_state_in),
                        static_cast<const void*>(conv_state_out), static_cast<const void*>(ssm_state_out)})
    if (!aligned(p, 4)) return fail(MAMBA_ERR_ALIGN, "float32 pointers must be 4-byte aligned");

  const size_t bld = static_cast<size_t>(batch) * seqlen * d_inner * es;
  // B and C: the last row ends d_state elements past its start
  const size_t bln = ((static_cast<size_t>(batch) * seqlen - 1) * bc_stride + d_state) * es;
  const size_t conv_bytes = static_cast<size_t>(batch) * d_inner * (d_conv - 1) * 4;
  const size_t ssm_bytes = static_cast<size_t>(batch) * d_inner * d_state * 4;
  const mscan::FwdPlan plan = (want_ckpt || want_dtp)
                                  ? mscan::plan_fwd_row(batch, seqlen, d_inner, io_dtype)
                                  : mscan::plan_fwd(batch, seqlen, d_inner, d_state, io_dtype, forced_kind);
  if (want_seq && plan.kind == mscan::kFwdChannel)
    return fail(MAMBA_ERR_SHAPE, "the lane-per-channel kernel has no document resets");
  if (xc_input && plan.kind == mscan::kFwdChannel)
    return fail(MAMBA_ERR_SHAPE, "the lane-per-channel kernel takes no xc input");
  const size_t ws_need = plan.ws_floats * sizeof(float);
  if (noalloc && ws_need > mscan::noalloc_scratch_bytes())
    return fail(MAMBA_ERR_WORKSPACE,
                "this shape needs %zu bytes of workspace; the fixed device scratch of mamba_scan_fwd_noalloc "
                "holds %zu (use mamba_scan_fwd with a caller workspace)",
                ws_need, mscan::noalloc_scratch_bytes());
  const size_t seq_bytes = want_seq ? static_cast<size_t>(batch) * seqlen * 4 : 0;
  // dt_low: the last row ends dt_rank elements past its start
  const size_t dtl_bytes = want_dtp ? ((static_cast<size_t>(batch) * seqlen - 1) * dtl_stride + dt_rank) * es : 0;
  // z: rows z_stride apart, the last ending d_inner elements past its start
  const size_t zn = ((static_cast<size_t>(batch) * seqlen - 1) * z_stride + d_inner) * es;
  const Range ins[] = {range("seq_idx", want_seq ? seq_idx : nullptr, seq_bytes),
                       range("x", x, bld), want_dtp ? range("dt_low", dt_low, dtl_bytes) : range("dt", dt, bld),
                       range("z", z, zn), range("B", B, bln),
                       range("C", C, bln), range("conv_w", conv_w, static_cast<size_t>(d_inner) * d_conv * 4),
                       range("conv_b", conv_b, static_cast<size_t>(d_inner) * 4),
                       range("dt_bias", dt_bias, static_cast<size_t>(d_inner) * 4),
                       range("D", D, static_cast<size_t>(d_inner) * 4),
                       range("A", A, static_cast<size_t>(d_inner) * d_state * 4),
                       range("conv_state_in", conv_state_in, conv_bytes),
                       range("ssm_state_in", ssm_state_in, ssm_bytes),
                       range("w_dt", want_dtp ? w_dt : nullptr,
                             want_dtp ? static_cast<size_t>(d_inner) * dt_rank * es : 0)};
  const Range outs[] = {range("y", y, bld), range("conv_state_out", conv_state_out, conv_bytes),
                        range("ssm_state_out", ssm_state_out, ssm_bytes),
                        range("workspace", ws_need ? workspace : nullptr, ws_need),
                        range("ckpt", want_ckpt ? ckpt : nullptr,
                              want_ckpt ? mscan::ckpt_floats(batch, seqlen, d_inner) * 4 : 0)};
  const Range pin[] = {range("conv_state_in", conv_state_in, conv_bytes),
                       range("ssm_state_in", ssm_state_in, ssm_bytes)};
  const Range pout[] = {range("conv_state_out", conv_state_out, conv_bytes),
                        range("ssm_state_out", ssm_state_out, ssm_bytes)};
  st = check_alias(ins, 14, outs, 5, pin, pout, 2);
  if (st) return st;
  // the outputs must not overlap one another either (ckpt against the rest)
  if (want_ckpt)
    for (int i = 0; i < 4; ++i)
      if (overlaps(outs[4], outs[i])) return fail(MAMBA_ERR_ALIAS, "ckpt overlaps output %s", outs[i].name);
  if (ws_need && !noalloc) {
    if (!workspace) return fail(MAMBA_ERR_WORKSPACE, "workspace is NULL but %zu bytes are required", ws_need);
    if (workspace_bytes < ws_need)
      return fail(MAMBA_ERR_WORKSPACE, "workspace has %zu bytes, %zu required", workspace_bytes, ws_need);
    if (!aligned(workspace, 4)) return fail(MAMBA_ERR_ALIGN, "workspace must be 4-byte aligned");
  }
  st = check_device();
  if (st) return st;
  if (noalloc) {  // the library's own device array (no caller memory can overlap it)
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = mscan::noalloc_scratch(dev, &workspace);
    if (e != hipSuccess) return fail(MAMBA_ERR_DEVICE, "device scratch lookup failed: %s", hipGetErrorString(e));
  }

  mscan::FwdCall c{batch, seqlen, d_inner, d_state, io_dtype, x, dt, z, B, C,
                   want_seq ? seq_idx : nullptr, conv_w, conv_b, dt_bias, D, A,
                   conv_state_in, ssm_state_in, y, conv_state_out, ssm_state_out,
                   static_cast<float*>(workspace), static_cast<hipStream_t>(stream), want_ckpt ? ckpt : nullptr,
                   force_wide, xc_input, bc_stride};
  if (want_dtp) {
    c.dt_low = dt_low;
    c.dtl_stride = dtl_stride;
    c.w_dt = w_dt;
    c.dt_rank = dt_rank;
    c.z_stride = z_stride;
  }
  const hipError_t err = mscan::launch_fwd(c, plan);
  if (err != hipSuccess) return fail(MAMBA_ERR_DEVICE, "kernel launch failed: %s", hipGetErrorString(err));
  g_calls.fetch_add(1);
  return ok();
}

}  // namespace

int mamba_scan_fwd(int32_t batch, int32_t seqlen, int32_t d_inner, int32_t d_state, int32_t d_conv,
                   int32_t io_dtype, const void* x, const void* dt, const void* z, const void* B, const void* C,
                   const float* conv_w, const float* conv_b, const float* dt_bias, const float* D, const float* A,
                   const float* conv_state_in, const float* ssm_state_in, void* y, float* conv_state_out,
                   float* ssm_state_out, void* workspace, size_t workspace_bytes, void* stream) {
  return fwd_common(batch, seqlen, d_inner, d_state, d_conv, io_dtype, x, dt, z, B, C, nullptr, false, conv_w,
                    conv_b, dt_bias, D, A, conv_state_in, ssm_state_in, y, conv_state_out, ssm_state_out, nullptr,
                    false, workspace, workspace_bytes, stream);
}

int mamba_scan_fwd_ckpt(int32_t batch, int32_t seqlen, int32_t d_inner, int32_t d_state, int32_t d_conv,
                        int32_t io_dtype, const void* x, const void* dt, const void* z, const void* B, const void* C,
                        const float* conv_w, const float* conv_b, const float* dt_bias, const float* D,
                        const float* A, const float* conv_state_in, const float* ssm_state_in, void* y,
                        float* conv_state_out, float* ssm_state_out, float* ckpt, void* workspace,
                        size_t workspace_bytes, void* stream) {
  return fwd_common(batch, seqlen, d_inner, d_state, d_conv, io_dtype, x, dt, z, B, C, nullptr, false, conv_w,
                    conv_b, dt_bias, D, A, conv_state_in, ssm_state_in, y, conv_state_out, ssm_state_out, ckpt, true,
                    workspace, workspace_bytes, stream);
}

int mamba_scan_fwd_seq(int32_t batch, int32_t seqlen, int32_t d_inner, int32_t d_state, int32_t d_conv,
                       int32_t io_dtype, const void* x, const void* dt, const void* z, const void* B,
                       const void* C, const int32_t* seq_idx, const float* conv_w, const float* conv_b,
                       const float* dt_bias, const float* D, const float* A, const float* conv_state_in,
                       const float* ssm_state_in, void* y, float* conv_state_out, float* ssm_state_out,
                       void* workspace, size_t workspace_bytes, void* stream) {
  return fwd_common(batch, seqlen, d_inner, d_state, d_conv, io_dtype, x, dt, z, B, C, seq_idx, true, conv_w,
                    conv_b, dt_bias, D, A, conv_state_in, ssm_state_in, y, conv_state_out, ssm_state_out, nullptr,
                    false, workspace, workspace_bytes, stream);
}

size_t mamba_scan_testing_fwd_workspace_bytes(int32_t kind, int32_t batch, int32_t seqlen, int32_t d_inner,
                                              int32_t d_state, int32_t io_dtype) {
  if (kind < -1 || kind > 2) return 0;
  if (batch < 1 || seqlen < 1 || d_inner < 1 || d_inner > (1 << 24) || (d_state != 8 && d_state != 16)) return 0;
  if (io_dtype != MAMBA_F32 && io_dtype != MAMBA_BF16) return 0;
  const int64_t widest = d_inner > d_state ? d_inner : d_state;
  if (!below_2_31({batch, seqlen, widest})) return 0;
  const size_t forced = mscan::plan_fwd(batch, seqlen, d_inner, d_state, io_dtype, kind).ws_floats;
  const size_t row = d_state == 16 ? mscan::plan_fwd_row(batch, seqlen, d_inner, io_dtype).ws_floats : 0;
  return (forced > row ? forced : row) * sizeof(float);
}

int mamba_scan_testing_fwd(int32_t kind, int32_t force_wide, int32_t batch, int32_t seqlen, int32_t d_inner,
                           int32_t d_state, int32_t d_conv, int32_t io_dtype, const void* x, const void* dt,
                           const void* z, const void* B, const void* C, const int32_t* seq_idx,
                           const float* conv_w, const float* conv_b, const float* dt_bias, const float* D,
                           const float* A, const float* conv_state_in, const float* ssm_state_in, void* y,
                           float* conv_state_out, float* ssm_state_out, float* ckpt, void* workspace,
                           size_t workspace_bytes, void* stream) {
  if (kind < -1 || kind > 2) return fail(MAMBA_ERR_SHAPE, "kind must be -1 (planned), 0, 1 or 2 (got %d)", kind);
  if (ckpt && seq_idx) return fail(MAMBA_ERR_SHAPE, "checkpoints are not produced over packed documents");
  if (ckpt && kind >= 0 && kind != 2) return fail(MAMBA_ERR_SHAPE, "checkpoints come from the row kernel (kind 2)");
  return fwd_common(batch, seqlen, d_inner, d_state, d_conv, io_dtype, x, dt, z, B, C, seq_idx, seq_idx != nullptr,
                    conv_w, conv_b, dt_bias, D, A, conv_state_in, ssm_state_in, y, conv_state_out, ssm_state_out,
                    ckpt, ckpt != nullptr, workspace, workspace_bytes, stream, kind, force_wide != 0);
}

int mamba_scan_fwd_xc(int32_t batch, int32_t seqlen, int32_t d_inner, int32_t d_state, int32_t io_dtype,
                      const void* xc, const void* dt, const void* z, const void* B, const void* C, int32_t bc_stride,
                      const float* dt_bias, const float* D, const float* A, const float* ssm_state_in, void* y,
                      float* ssm_state_out, void* workspace, size_t workspace_bytes, void* stream) {
  if (bc_stride < 1) return fail(MAMBA_ERR_SHAPE, "bc_stride must be >= d_state (got %d)", bc_stride);
  return fwd_common(batch, seqlen, d_inner, d_state, 4, io_dtype, xc, dt, z, B, C, nullptr, false, nullptr, nullptr,
                    dt_bias, D, A, nullptr, ssm_state_in, y, nullptr, ssm_state_out, nullptr, false, workspace,
                    workspace_bytes, stream, -1, false, false, true, bc_stride);
}

int mamba_scan_fwd_xc_dtproj(int32_t batch, int32_t seqlen, int32_t d_inner, int32_t d_state, int32_t dt_rank,
                             int32_t io_dtype, const void* xc, const void* dt_low, int32_t dtl_stride,
                             const void* w_dt, const void* z, int32_t z_stride, const void* B, const void* C,
                             int32_t bc_stride, const float* dt_bias, const float* D, const float* A,
                             const float* ssm_state_in, void* y, float* ssm_state_out, void* workspace,
                             size_t workspace_bytes, void* stream) {
  if (bc_stride < 1) return fail(MAMBA_ERR_SHAPE, "bc_stride must be >= d_state (got %d)", bc_stride);
  if (z_stride < 1) return fail(MAMBA_ERR_SHAPE, "z_stride must be >= d_inner (got %d)", z_stride);
  return fwd_common(batch, seqlen, d_inner, d_state, 4, io_dtype, xc, nullptr, z, B, C, nullptr, false, nullptr,
                    nullptr, dt_bias, D, A, nullptr, ssm_state_in, y, nullptr, ssm_state_out, nullptr, false,
                    workspace, workspace_bytes, stream, -1, false, false, true, bc_stride, true, dt_low, dtl_stride,
                    w_dt, dt_rank, z_stride);
}

int mamba_scan_fwd_noalloc(int32_t batch, int32_t seqlen, int32_t d_inner, int32_t d_state, int32_t d_conv,
                           int32_t io_dtype, const void* x, const void* dt, const void* z, const void* B,
                           const void* C, const float* conv_w, const float* conv_b, const float* dt_bias,
                           const float* D, const float* A, const float* conv_state_in, const float* ssm_state_in,
                           void* y, float* conv_state_out, float* ssm_state_out, void* stream) {
  return fwd_common(batch, seqlen, d_inner, d_state, d_conv, io_dtype, x, dt, z, B, C, nullptr, false, conv_w,
                    conv_b, dt_bias, D, A, conv_state_in, ssm_state_in, y, conv_state_out, ssm_state_out, nullptr,
                    false, nullptr, 0, stream, -1, false, true);
}

size_t mamba_scan_bwd_workspace_bytes(int32_t batch, int32_t seqlen, int32_t d_inner, int32_t d_state,
                                      int32_t io_dtype) {
  if (batch < 1 || seqlen < 1 || d_inner < 1 || d_inner > (1 << 24) || d_state != 16) return 0;
  if (io_dtype != MAMBA_F32 && io_dtype != MAMBA_BF16) return 0;
  if (!below_2_31({batch, (d_inner + 15) / 16, 128}) || !below_2_31({batch, seqlen, 8})) return 0;
  if (!below_2_31({batch, seqlen, d_inner})) return 0;
  return mscan::bwd_ws_layout(batch, seqlen, d_inner).total * sizeof(float);
}

size_t mamba_scan_bwd_ckpt_workspace_bytes(int32_t batch, int32_t seqlen, int32_t d_inner, int32_t d_state,
                                           int32_t io_dtype) {
  if (mamba_scan_bwd_workspace_bytes(batch, seqlen, d_inner, d_state, io_dtype) == 0) return 0;
  return mscan::bwd_ws_layout(batch, seqlen, d_inner, false).total * sizeof(float);
}

namespace {

int bwd_common(int32_t batch, int32_t seqlen, int32_t d_inner, int32_t d_state, int32_t d_conv, int32_t io_dtype,
               const void* x, const void* dt, const void* z, const void* B, const void* C, const float* conv_w,
               const float* conv_b, const float* dt_bias, const float* D, const float* A,
               const float* conv_state_in, const float* ssm_state_in, const void* dy, void* dx, void* ddt, void* dz,
               float* dB, float* dC, float* dconv_w, float* dconv_b, float* ddt_bias, float* dD, float* dA,
               const float* ckpt, bool want_ckpt, void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_dims(batch, seqlen, d_inner, d_state, d_conv);
  if (st) return st;
  if (d_state != 16) return fail(MAMBA_ERR_SHAPE, "the backward serves d_state 16 only (got %d)", d_state);
  if (d_inner > (1 << 24))  // per-lane byte offsets within a stage's rows must stay below 2^31
    return fail(MAMBA_ERR_SHAPE, "the backward serves d_inner <= 2^24 (got %d)", d_inner);
  // A dispatch counts the work-items of each grid dimension in 32 bits: the
  // sequential kernels launch batch * ceil(d_inner / 16) workgroups of 256,
  // and the dB/dC reduction 16 threads per (batch row, timestep).
  if (!below_2_31({batch, (d_inner + 15) / 16, 128}))
    return fail(MAMBA_ERR_SHAPE, "the backward needs batch * ceil(d_inner / 16) < 2^24 (got %d x %d)", batch,
                (d_inner + 15) / 16);
  if (!below_2_31({batch, seqlen, 8}))
    return fail(MAMBA_ERR_SHAPE, "the backward needs batch * seqlen < 2^28 (got %d x %d)", batch, seqlen);
  if (io_dtype != MAMBA_F32 && io_dtype != MAMBA_BF16)
    return fail(MAMBA_ERR_DTYPE, "io_dtype must be MAMBA_F32 (0) or MAMBA_BF16 (1), got %d", io_dtype);
  const struct { const void* p; const char* n; } req[] = {
      {x, "x"}, {dt, "dt"}, {z, "z"}, {B, "B"}, {C, "C"}, {conv_w, "conv_w"}, {conv_b, "conv_b"},
      {dt_bias, "dt_bias"}, {D, "D"}, {A, "A"}, {dy, "dy"}, {dx, "dx"}, {ddt, "ddt"}, {dz, "dz"}, {dB, "dB"},
      {dC, "dC"}, {dconv_w, "dconv_w"}, {dconv_b, "dconv_b"}, {ddt_bias, "ddt_bias"}, {dD, "dD"}, {dA, "dA"}};
  for (const auto& r : req)
    if (!r.p) return fail(MAMBA_ERR_NULL, "%s is NULL", r.n);
  if (want_ckpt && !ckpt) return fail(MAMBA_ERR_NULL, "ckpt is NULL");
  const size_t es = io_size(io_dtype);
  for (const void* p : {x, dt, z, B, C, dy, static_cast<const void*>(dx), static_cast<const void*>(ddt),
                        static_cast<const void*>(dz)})
    if (!aligned(p, es)) return fail(MAMBA_ERR_ALIGN, "io pointers must be %zu-byte aligned", es);
  for (const void* p : {static_cast<const void*>(conv_w), static_cast<const void*>(conv_b),
                        static_cast<const void*>(dt_bias), static_cast<const void*>(D), static_cast<const void*>(A),
                        static_cast<const void*>(conv_state_in), static_cast<const void*>(ssm_state_in),
                        static_cast<const void*>(dB), static_cast<const void*>(dC), static_cast<const void*>(dconv_w),
                        static_cast<const void*>(dconv_b), static_cast<const void*>(ddt_bias),
                        static_cast<const void*>(dD), static_cast<const void*>(dA), static_cast<const void*>(ckpt)})
    if (!aligned(p, 4)) return fail(MAMBA_ERR_ALIGN, "float32 pointers must be 4-byte aligned");
  const size_t bld = static_cast<size_t>(batch) * seqlen * d_inner * es;
  const size_t bln = static_cast<size_t>(batch) * seqlen * d_state * es;
  const size_t bln4 = static_cast<size_t>(batch) * seqlen * d_state * 4;
  const size_t dv = static_cast<size_t>(d_inner) * 4;
  const size_t ws_need = mscan::bwd_ws_layout(batch, seqlen, d_inner, !want_ckpt).total * sizeof(float);
  const Range ins[] = {range("x", x, bld), range("dt", dt, bld), range("z", z, bld), range("B", B, bln),
                       range("C", C, bln), range("conv_w", conv_w, dv * 4), range("conv_b", conv_b, dv),
                       range("dt_bias", dt_bias, dv), range("D", D, dv), range("A", A, dv * d_state),
                       range("conv_state_in", conv_state_in, static_cast<size_t>(batch) * d_inner * 3 * 4),
                       range("ssm_state_in", ssm_state_in, static_cast<size_t>(batch) * d_inner * d_state * 4),
                       range("dy", dy, bld),
                       range("ckpt", want_ckpt ? ckpt : nullptr,
                             want_ckpt ? mscan::ckpt_floats(batch, seqlen, d_inner) * 4 : 0)};
  const Range outs[] = {range("dx", dx, bld), range("ddt", ddt, bld), range("dz", dz, bld), range("dB", dB, bln4),
                        range("dC", dC, bln4), range("dconv_w", dconv_w, dv * 4), range("dconv_b", dconv_b, dv),
                        range("ddt_bias", ddt_bias, dv), range("dD", dD, dv), range("dA", dA, dv * d_state),
                        range("workspace", workspace, ws_need)};
  st = check_alias(ins, 14, outs, 11, nullptr, nullptr, 0);
  if (st) return st;
  if (!workspace) return fail(MAMBA_ERR_WORKSPACE, "workspace is NULL but %zu bytes are required", ws_need);
  if (workspace_bytes < ws_need)
    return fail(MAMBA_ERR_WORKSPACE, "workspace has %zu bytes, %zu required", workspace_bytes, ws_need);
  if (!aligned(workspace, 16)) return fail(MAMBA_ERR_ALIGN, "workspace must be 16-byte aligned");
  st = check_device();
  if (st) return st;
  mscan::BwdCall c{batch, seqlen, d_inner, d_state, io_dtype, x, dt, z, B, C, conv_w, conv_b, dt_bias, D, A,
                   conv_state_in, ssm_state_in, dy, dx, ddt, dz, dB, dC, dconv_w, dconv_b, ddt_bias, dD, dA,
                   static_cast<float*>(workspace), static_cast<hipStream_t>(stream), want_ckpt ? ckpt : nullptr};
  const hipError_t err = mscan::launch_bwd(c);
  if (err != hipSuccess) return fail(MAMBA_ERR_DEVICE, "kernel launch failed: %s", hipGetErrorString(err));
  g_calls.fetch_add(1);
  return ok();
}

}  // namespace

int mamba_scan_bwd(int32_t batch, int32_t seqlen, int32_t d_inner, int32_t d_state, int32_t d_conv,
                   int32_t io_dtype, const void* x, const void* dt, const void* z, const void* B, const void* C,
                   const float* conv_w, const float* conv_b, const float* dt_bias, const float* D, const float* A,
                   const float* conv_state_in, const float* ssm_state_in, const void* dy, void* dx, void* ddt,
                   void* dz, float* dB, float* dC, float* dconv_w, float* dconv_b, float* ddt_bias, float* dD,
                   float* dA, void* workspace, size_t workspace_bytes, void* stream) {
  return bwd_common(batch, seqlen, d_inner, d_state, d_conv, io_dtype, x, dt, z, B, C, conv_w, conv_b, dt_bias, D,
                    A, conv_state_in, ssm_state_in, dy, dx, ddt, dz, dB, dC, dconv_w, dconv_b, ddt_bias, dD, dA,
                    nullptr, false, workspace, workspace_bytes, stream);
}

int mamba_scan_bwd_ckpt(int32_t batch, int32_t seqlen, int32_t d_inner, int32_t d_state, int32_t d_conv,
                        int32_t io_dtype, const void* x, const void* dt, const void* z, const void* B, const void* C,
                        const float* conv_w, const float* conv_b, const float* dt_bias, const float* D,
                        const float* A, const float* conv_state_in, const float* ssm_state_in, const void* dy,
                        void* dx, void* ddt, void* dz, float* dB, float* dC, float* dconv_w, float* dconv_b,
                        float* ddt_bias, float* dD, float* dA, const float* ckpt, void* workspace,
                        size_t workspace_bytes, void* stream) {
  return bwd_common(batch, seqlen, d_inner, d_state, d_conv, io_dtype, x, dt, z, B, C, conv_w, conv_b, dt_bias, D,
                    A, conv_state_in, ssm_state_in, dy, dx, ddt, dz, dB, dC, dconv_w, dconv_b, ddt_bias, dD, dA,
                    ckpt, true, workspace, workspace_bytes, stream);
}

namespace {

int check_ssd_dims(int32_t batch, int32_t seqlen, int32_t nheads, int32_t headdim, int32_t d_state,
                   int32_t ngroups) {
  if (batch < 1 || seqlen < 1 || nheads < 1 || ngroups < 1)
    return fail(MAMBA_ERR_SHAPE, "dims must be >= 1 (batch=%d seqlen=%d nheads=%d ngroups=%d)", batch, seqlen,
                nheads, ngroups);
  if (headdim != 64) return fail(MAMBA_ERR_SHAPE, "headdim must be 64 (got %d)", headdim);
  if (d_state != 64 && d_state != 128) return fail(MAMBA_ERR_SHAPE, "d_state must be 64 or 128 (got %d)", d_state);
  if (nheads % ngroups != 0)
    return fail(MAMBA_ERR_SHAPE, "ngroups (%d) must divide nheads (%d)", ngroups, nheads);
  if (batch > 65535 || nheads > 65535)
    return fail(MAMBA_ERR_SHAPE, "batch and nheads must be <= 65535 (got %d, %d)", batch, nheads);
  if (!below_2_31({batch, seqlen, nheads, headdim}) || !below_2_31({batch, seqlen, ngroups, d_state}))
    return fail(MAMBA_ERR_SHAPE, "tensor too large (batch*seqlen*nheads*headdim must be < 2^31)");
  return MAMBA_OK;
}

}  // namespace

size_t mamba2_ssd_fwd_workspace_bytes(int32_t batch, int32_t seqlen, int32_t nheads, int32_t headdim,
                                      int32_t d_state, int32_t ngroups, int32_t io_dtype) {
  if (io_dtype != MAMBA_F32 && io_dtype != MAMBA_BF16) return 0;
  const std::string saved = g_last_error;
  const int st = check_ssd_dims(batch, seqlen, nheads, headdim, d_state, ngroups);
  g_last_error = saved;
  if (st) return 0;
  return mscan::ssd_ws_layout(batch, seqlen, nheads, d_state).total * sizeof(float);
}

namespace {

int ssd_fwd_common(int32_t batch, int32_t seqlen, int32_t nheads, int32_t headdim, int32_t d_state,
                   int32_t ngroups, int32_t io_dtype, const void* x, const void* dt, const void* B, const void* C,
                   const int32_t* seq_idx, bool want_seq, const float* dt_bias, const float* A, const float* D,
                   const float* state_in, void* y, float* state_out, void* workspace, size_t workspace_bytes,
                   void* stream) {
  int st = check_ssd_dims(batch, seqlen, nheads, headdim, d_state, ngroups);
  if (st) return st;
  if (io_dtype != MAMBA_F32 && io_dtype != MAMBA_BF16)
    return fail(MAMBA_ERR_DTYPE, "io_dtype must be MAMBA_F32 (0) or MAMBA_BF16 (1), got %d", io_dtype);
  const struct { const void* p; const char* n; } req[] = {{x, "x"}, {dt, "dt"}, {B, "B"}, {C, "C"},
                                                          {dt_bias, "dt_bias"}, {A, "A"}, {D, "D"}, {y, "y"}};
  for (const auto& r : req)
    if (!r.p) return fail(MAMBA_ERR_NULL, "%s is NULL", r.n);
  if (want_seq && !seq_idx) return fail(MAMBA_ERR_NULL, "seq_idx is NULL");
  if (want_seq && !aligned(seq_idx, 4)) return fail(MAMBA_ERR_ALIGN, "seq_idx must be 4-byte aligned");
  const size_t es = io_size(io_dtype);
  for (const void* p : {x, B, C, static_cast<const void*>(y)})
    if (!aligned(p, 16)) return fail(MAMBA_ERR_ALIGN, "x, B, C and y must be 16-byte aligned");
  if (!aligned(dt, es)) return fail(MAMBA_ERR_ALIGN, "dt must be %zu-byte aligned", es);
  for (const void* p : {static_cast<const void*>(dt_bias), static_cast<const void*>(A), static_cast<const void*>(D)})
    if (!aligned(p, 4)) return fail(MAMBA_ERR_ALIGN, "float32 parameters must be 4-byte aligned");
  if (!aligned(state_in, 16) || !aligned(state_out, 16))
    return fail(MAMBA_ERR_ALIGN, "state_in and state_out must be 16-byte aligned");
  const size_t rows = static_cast<size_t>(batch) * seqlen;
  const size_t bx = rows * nheads * headdim * es, bdt = rows * nheads * es, bbc = rows * ngroups * d_state * es;
  const size_t bpar = static_cast<size_t>(nheads) * 4;
  const size_t bst = static_cast<size_t>(batch) * nheads * headdim * d_state * 4;
  const size_t ws_need = mscan::ssd_ws_layout(batch, seqlen, nheads, d_state).total * sizeof(float);
  const Range ins[] = {range("x", x, bx), range("dt", dt, bdt), range("B", B, bbc), range("C", C, bbc),
                       range("dt_bias", dt_bias, bpar), range("A", A, bpar), range("D", D, bpar),
                       range("state_in", state_in, bst), range("seq_idx", want_seq ? seq_idx : nullptr, rows * 4)};
  const Range outs[] = {range("y", y, bx), range("state_out", state_out, bst),
                        range("workspace", workspace, ws_need)};
  const Range pin[] = {range("state_in", state_in, bst)};
  const Range pout[] = {range("state_out", state_out, bst)};
  st = check_alias(ins, 9, outs, 3, pin, pout, 1);
  if (st) return st;
  if (!workspace) return fail(MAMBA_ERR_WORKSPACE, "workspace is NULL but %zu bytes are required", ws_need);
  if (workspace_bytes < ws_need)
    return fail(MAMBA_ERR_WORKSPACE, "workspace has %zu bytes, %zu required", workspace_bytes, ws_need);
  if (!aligned(workspace, 256)) return fail(MAMBA_ERR_ALIGN, "workspace must be 256-byte aligned");
  st = check_device();
  if (st) return st;
  mscan::SsdCall c{batch, seqlen, nheads, headdim, d_state, ngroups, io_dtype, x, dt, B, C,
                   want_seq ? seq_idx : nullptr, dt_bias, A, D, state_in, y, state_out,
                   static_cast<float*>(workspace), static_cast<hipStream_t>(stream)};
  const hipError_t err = mscan::launch_ssd(c);
  if (err != hipSuccess) return fail(MAMBA_ERR_DEVICE, "kernel launch failed: %s", hipGetErrorString(err));
  g_calls.fetch_add(1);
  return ok();
}

}  // namespace

int mamba2_ssd_fwd(int32_t batch, int32_t seqlen, int32_t nheads, int32_t headdim, int32_t d_state, int32_t ngroups,
                   int32_t io_dtype, const void* x, const void* dt, const void* B, const void* C,
                   const float* dt_bias, const float* A, const float* D, const float* state_in, void* y,
                   float* state_out, void* workspace, size_t workspace_bytes, void* stream) {
  return ssd_fwd_common(batch, seqlen, nheads, headdim, d_state, ngroups, io_dtype, x, dt, B, C, nullptr, false,
                        dt_bias, A, D, state_in, y, state_out, workspace, workspace_bytes, stream);
}

int mamba2_ssd_fwd_seq(int32_t batch, int32_t seqlen, int32_t nheads, int32_t headdim, int32_t d_state,
                       int32_t ngroups, int32_t io_dtype, const void* x, const void* dt, const void* B,
                       const void* C, const int32_t* seq_idx, const float* dt_bias, const float* A, const float* D,
                       const float* state_in, void* y, float* state_out, void* workspace, size_t workspace_bytes,
                       void* stream) {
  return ssd_fwd_common(batch, seqlen, nheads, headdim, d_state, ngroups, io_dtype, x, dt, B, C, seq_idx, true,
                        dt_bias, A, D, state_in, y, state_out, workspace, workspace_bytes, stream);
}

int mamba2_ssd_step(int32_t batch, int32_t nheads, int32_t headdim, int32_t d_state, int32_t ngroups,
                    int32_t io_dtype, const void* x, const void* dt, const void* B, const void* C,
                    const float* dt_bias, const float* A, const float* D, const float* state_in, void* y,
                    float* state_out, void* stream) {
  int st = check_ssd_dims(batch, 1, nheads, headdim, d_state, ngroups);
  if (st) return st;
  if (io_dtype != MAMBA_F32 && io_dtype != MAMBA_BF16)
    return fail(MAMBA_ERR_DTYPE, "io_dtype must be MAMBA_F32 (0) or MAMBA_BF16 (1), got %d", io_dtype);
  const struct { const void* p; const char* n; } req[] = {
      {x, "x"}, {dt, "dt"}, {B, "B"}, {C, "C"}, {dt_bias, "dt_bias"}, {A, "A"}, {D, "D"},
      {state_in, "state_in"}, {y, "y"}, {state_out, "state_out"}};
  for (const auto& r : req)
    if (!r.p) return fail(MAMBA_ERR_NULL, "%s is NULL", r.n);
  const size_t es = io_size(io_dtype);
  for (const void* p : {x, dt, B, C, static_cast<const void*>(y)})
    if (!aligned(p, es)) return fail(MAMBA_ERR_ALIGN, "io pointers must be %zu-byte aligned", es);
  for (const void* p : {static_cast<const void*>(dt_bias), static_cast<const void*>(A), static_cast<const void*>(D)})
    if (!aligned(p, 4)) return fail(MAMBA_ERR_ALIGN, "float32 parameters must be 4-byte aligned");
  if (!aligned(state_in, 16) || !aligned(state_out, 16))
    return fail(MAMBA_ERR_ALIGN, "state_in and state_out must be 16-byte aligned");
  const size_t bx = static_cast<size_t>(batch) * nheads * headdim * es, bdt = static_cast<size_t>(batch) * nheads * es;
  const size_t bbc = static_cast<size_t>(batch) * ngroups * d_state * es, bpar = static_cast<size_t>(nheads) * 4;
  const size_t bst = static_cast<size_t>(batch) * nheads * headdim * d_state * 4;
  const Range ins[] = {range("x", x, bx), range("dt", dt, bdt), range("B", B, bbc), range("C", C, bbc),
                       range("dt_bias", dt_bias, bpar), range("A", A, bpar), range("D", D, bpar),
                       range("state_in", state_in, bst)};
  const Range outs[] = {range("y", y, bx), range("state_out", state_out, bst)};
  const Range pin[] = {range("state_in", state_in, bst)};
  const Range pout[] = {range("state_out", state_out, bst)};
  st = check_alias(ins, 8, outs, 2, pin, pout, 1);
  if (st) return st;
  st = check_device();
  if (st) return st;
  mscan::SsdCall c{batch, 1, nheads, headdim, d_state, ngroups, io_dtype, x, dt, B, C, nullptr, dt_bias, A, D,
                   state_in, y, state_out, nullptr, static_cast<hipStream_t>(stream)};
  const hipError_t err = mscan::launch_ssd_step(c);
  if (err != hipSuccess) return fail(MAMBA_ERR_DEVICE, "kernel launch failed: %s", hipGetErrorString(err));
  g_calls.fetch_add(1);
  return ok();
}

namespace {

// One token; with xc_input, x holds the activated conv output and the conv
// weights and states are absent (NULL) and untouched.
int step_common(int32_t batch, int32_t d_inner, int32_t d_state, int32_t d_conv, int32_t io_dtype, const void* x,
                const void* dt, const void* z, const void* B, const void* C, const float* conv_w,
                const float* conv_b, const float* dt_bias, const float* D, const float* A,
                const float* conv_state_in, const float* ssm_state_in, void* y, float* conv_state_out,
                float* ssm_state_out, void* stream, bool xc_input, int32_t bc_stride,
                const void* dt_low = nullptr, int32_t dtl_stride = 0, const void* w_dt = nullptr,
                int32_t dt_rank = 0, int32_t z_stride = 0) {
  int st = check_dims(batch, 1, d_inner, d_state, d_conv);
  if (st) return st;
  const bool dtp = dt_low != nullptr || w_dt != nullptr || dt_rank != 0;  // dt_proj inside (xc input only)
  if (z_stride == 0) z_stride = d_inner;  // contiguous z
  if (z_stride != d_inner) {               // z read from wider rows (with dt_proj inside)
    if (z_stride < d_inner || z_stride > kMaxBcStride)
      return fail(MAMBA_ERR_SHAPE, "z_stride (%d) must lie in [d_inner, 2^24] (d_inner %d)", z_stride, d_inner);
    if (!below_2_31({batch, z_stride})) return fail(MAMBA_ERR_SHAPE, "batch * z_stride must be below 2^31");
  }
  if (dtp) {
    if (dt_rank < 1 || dt_rank > kMaxDtRank)
      return fail(MAMBA_ERR_SHAPE, "dt_rank must lie in [1, %d] (got %d)", kMaxDtRank, dt_rank);
    if (dtl_stride < dt_rank || dtl_stride > kMaxBcStride)
      return fail(MAMBA_ERR_SHAPE, "dt_low's row stride (%d) must lie in [dt_rank, 2^24]", dtl_stride);
    if (!below_2_31({batch, dtl_stride})) return fail(MAMBA_ERR_SHAPE, "batch * dtl_stride must be below 2^31");
    if (!dt_low) return fail(MAMBA_ERR_NULL, "dt_low is NULL");
    if (!w_dt) return fail(MAMBA_ERR_NULL, "w_dt is NULL");
    dt = dt_low;  // stands in for the absent dt in the checks below (its own extent is checked separately)
  }
  if (bc_stride < d_state || bc_stride > kMaxBcStride)
    return fail(MAMBA_ERR_SHAPE, "bc_stride (%d) must lie in [d_state, 2^24] (d_state %d)", bc_stride, d_state);
  if (!below_2_31({batch, bc_stride})) return fail(MAMBA_ERR_SHAPE, "batch * bc_stride must be below 2^31");
  if (io_dtype != MAMBA_F32 && io_dtype != MAMBA_BF16)
    return fail(MAMBA_ERR_DTYPE, "io_dtype must be MAMBA_F32 (0) or MAMBA_BF16 (1), got %d", io_dtype);
  const void* no_conv = dt;  // stands in for the absent conv pointers of an xc input
  const struct { const void* p; const char* n; } req[] = {
      {x, xc_input ? "xc" : "x"}, {dt, "dt"}, {z, "z"}, {B, "B"}, {C, "C"},
      {xc_input ? no_conv : conv_w, "conv_w"}, {xc_input ? no_conv : conv_b, "conv_b"},
      {dt_bias, "dt_bias"}, {D, "D"}, {A, "A"}, {xc_input ? no_conv : conv_state_in, "conv_state_in"},
      {ssm_state_in, "ssm_state_in"}, {y, "y"}, {xc_input ? no_conv : conv_state_out, "conv_state_out"},
      {ssm_state_out, "ssm_state_out"}};
  for (const auto& r : req)
    if (!r.p) return fail(MAMBA_ERR_NULL, "%s is NULL", r.n);
  const size_t es = io_size(io_dtype);
  for (const void* p : {x, dt, z, B, C, static_cast<const void*>(y)})
    if (!aligned(p, es)) return fail(MAMBA_ERR_ALIGN, "io pointers must be %zu-byte aligned", es);
  for (const void* p : {static_cast<const void*>(conv_w), static_cast<const void*>(conv_b),
                        static_cast<const void*>(dt_bias), static_cast<const void*>(D), static_cast<const void*>(A),
                        static_cast<const void*>(conv_state_in), static_cast<const void*>(ssm_state_in),
                        static_cast<const void*>(conv_state_out), static_cast<const void*>(ssm_state_out)})
    if (!aligned(p, 4)) return fail(MAMBA_ERR_ALIGN, "float32 pointers must be 4-byte aligned");

  const size_t bd = static_cast<size_t>(batch) * d_inner * es;
  for (const void* p : {dt_low, w_dt})
    if (!aligned(p, es)) return fail(MAMBA_ERR_ALIGN, "io pointers must be %zu-byte aligned", es);
  const size_t bn = ((static_cast<size_t>(batch) - 1) * bc_stride + d_state) * es;  // B, C rows bc_stride apart
  const size_t dtl_bytes = dtp ? ((static_cast<size_t>(batch) - 1) * dtl_stride + dt_rank) * es : 0;
  const size_t wdt_bytes = dtp ? static_cast<size_t>(d_inner) * dt_rank * es : 0;
  const size_t conv_bytes = static_cast<size_t>(batch) * d_inner * (d_conv - 1) * 4;
  const size_t ssm_bytes = static_cast<size_t>(batch) * d_inner * d_state * 4;
  const size_t zn = ((static_cast<size_t>(batch) - 1) * z_stride + d_inner) * es;  // z rows z_stride apart
  const Range ins[] = {range("x", x, bd), range("dt", dtp ? nullptr : dt, bd), range("z", z, zn),
                       range("B", B, bn), range("C", C, bn),
                       range("conv_w", conv_w, static_cast<size_t>(d_inner) * d_conv * 4),
                       range("conv_b", conv_b, static_cast<size_t>(d_inner) * 4),
                       range("dt_bias", dt_bias, static_cast<size_t>(d_inner) * 4),
                       range("D", D, static_cast<size_t>(d_inner) * 4),
                       range("A", A, static_cast<size_t>(d_inner) * d_state * 4),
                       range("conv_state_in", conv_state_in, conv_bytes),
                       range("ssm_state_in", ssm_state_in, ssm_bytes), range("dt_low", dt_low, dtl_bytes),
                       range("w_dt", w_dt, wdt_bytes)};
  const Range outs[] = {range("y", y, bd), range("conv_state_out", conv_state_out, conv_bytes),
                        range("ssm_state_out", ssm_state_out, ssm_bytes)};
  const Range pin[] = {range("conv_state_in", conv_state_in, conv_bytes),
                       range("ssm_state_in", ssm_state_in, ssm_bytes)};
  const Range pout[] = {range("conv_state_out", conv_state_out, conv_bytes),
                        range("ssm_state_out", ssm_state_out, ssm_bytes)};
  st = check_alias(ins, 14, outs, 3, pin, pout, 2);
  if (st) return st;
  st = check_device();
  if (st) return st;

  mscan::StepCall c{batch, d_inner, d_state, io_dtype, x, dt, z, B, C, conv_w, conv_b, dt_bias, D, A,
                    conv_state_in, ssm_state_in, y, conv_state_out, ssm_state_out,
                    static_cast<hipStream_t>(stream), xc_input, bc_stride, dtp ? dt_low : nullptr, dtl_stride,
                    w_dt, dt_rank, z_stride};
  const hipError_t err = mscan::launch_step(c);
  if (err != hipSuccess) return fail(MAMBA_ERR_DEVICE, "kernel launch failed: %s", hipGetErrorString(err));
  g_calls.fetch_add(1);
  return ok();
}

}  // namespace

int mamba_scan_step(int32_t batch, int32_t d_inner, int32_t d_state, int32_t d_conv, int32_t io_dtype,
                    const void* x, const void* dt, const void* z, const void* B, const void* C,
                    const float* conv_w, const float* conv_b, const float* dt_bias, const float* D, const float* A,
                    const float* conv_state_in, const float* ssm_state_in, void* y, float* conv_state_out,
                    float* ssm_state_out, void* stream) {
  return step_common(batch, d_inner, d_state, d_conv, io_dtype, x, dt, z, B, C, conv_w, conv_b, dt_bias, D, A,
                     conv_state_in, ssm_state_in, y, conv_state_out, ssm_state_out, stream, false, d_state);
}

int mamba_scan_step_xc(int32_t batch, int32_t d_inner, int32_t d_state, int32_t io_dtype, const void* xc,
                       const void* dt, const void* z, const void* B, const void* C, int32_t bc_stride,
                       const float* dt_bias, const float* D, const float* A, const float* ssm_state_in, void* y,
                       float* ssm_state_out, void* stream) {
  return step_common(batch, d_inner, d_state, 4, io_dtype, xc, dt, z, B, C, nullptr, nullptr, dt_bias, D, A, nullptr,
                     ssm_state_in, y, nullptr, ssm_state_out, stream, true, bc_stride);
}

int mamba_scan_step_xc_dtproj(int32_t batch, int32_t d_inner, int32_t d_state, int32_t dt_rank, int32_t io_dtype,
                              const void* xc, const void* dt_low, int32_t dtl_stride, const void* w_dt,
                              const void* z, int32_t z_stride, const void* B, const void* C, int32_t bc_stride,
                              const float* dt_bias, const float* D, const float* A, const float* ssm_state_in,
                              void* y, float* ssm_state_out, void* stream) {
  if (dt_rank < 1) return fail(MAMBA_ERR_SHAPE, "dt_rank must be >= 1 (got %d)", dt_rank);
  if (z_stride < 1) return fail(MAMBA_ERR_SHAPE, "z_stride must be >= d_inner (got %d)", z_stride);
  return step_common(batch, d_inner, d_state, 4, io_dtype, xc, nullptr, z, B, C, nullptr, nullptr, dt_bias, D, A,
                     nullptr, ssm_state_in, y, nullptr, ssm_state_out, stream, true, bc_stride, dt_low, dtl_stride,
                     w_dt, dt_rank, z_stride);
}

}  // extern "C"
