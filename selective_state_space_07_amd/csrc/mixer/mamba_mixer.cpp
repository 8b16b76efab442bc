// C-ABI layer of libmamba_mixer: one Mamba-1 mixer layer (calm-mamba 0.1.4
// PKG-INFO, "Mamba operator", steps 1-7) as in_proj / x_proj / out_proj GEMMs
// (rocBLAS) around the selective-scan library's prefill and decode entry
// points, which also run dt_proj (a GEMM only for shapes the fused prefill
// does not take), with the conv + SiLU that feeds x_proj in a kernel of this
// library (declared in include/mamba_mixer.h).
#include "../../../include/mamba_mixer.h"

#include <hip/hip_runtime.h>
#include <rocblas/rocblas.h>

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "mixer_internal.h"

namespace {

thread_local std::string g_last_error;

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
size_t up256(size_t n) { return (n + 255) / 256 * 256; }
bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Offsets (bytes) of the intermediates in the workspace, for `tokens` rows.
// in_proj's output takes 2 * tokens * d_inner elements at x: one GEMM writes
// rows [tokens][2 * d_inner] (x, then z; the conv and the scan read them with
// that row stride), or, where the scan takes z contiguous only, two GEMMs
// write x [tokens][d_inner] and then z at offset z.
// x_proj's output xp [tokens][dt_rank + 2 * d_state] holds dt_low, B and C
// side by side: dt_proj and the scan read them in place (row stride
// dt_rank + 2 * d_state), so x_proj is one GEMM that reads xc once.
struct Layout {
  size_t x, z, xc, xp, dt, y, scan, total;
};

Layout layout(int64_t tokens, int32_t d_inner, int32_t d_state, int32_t dt_rank, size_t es, size_t scan_bytes) {
  Layout l{};
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o += up256(bytes);
    return at;
  };
  const size_t td = static_cast<size_t>(tokens) * d_inner * es;
  l.x = take(2 * td);
  l.z = l.x + td;
  l.xc = take(td);
  l.xp = take(static_cast<size_t>(tokens) * (dt_rank + 2 * d_state) * es);
  l.dt = take(td);
  l.y = take(td);
  l.scan = take(scan_bytes);
  l.total = o;
  return l;
}

int check_dims(int64_t tokens, int32_t d_model, int32_t d_inner, int32_t d_state, int32_t dt_rank, int32_t d_conv,
               int32_t io_dtype) {
  if (tokens < 1 || d_model < 1 || d_inner < 1 || dt_rank < 1)
    return fail(MAMBA_ERR_SHAPE, "dims must be >= 1 (tokens=%lld d_model=%d d_inner=%d dt_rank=%d)",
                static_cast<long long>(tokens), d_model, d_inner, dt_rank);
  if (d_conv != 4) return fail(MAMBA_ERR_SHAPE, "d_conv must be 4 (got %d)", d_conv);
  if (d_state != 8 && d_state != 16) return fail(MAMBA_ERR_SHAPE, "d_state must be 8 or 16 (got %d)", d_state);
  const int64_t widest = std::max<int64_t>(std::max<int64_t>(2LL * d_inner, d_model), dt_rank + 2LL * d_state);
  // tokens < 2^31 first, so the product (widest < 2^33) cannot overflow
  if (tokens >= (int64_t{1} << 31) || tokens * widest >= (int64_t{1} << 31))
    return fail(MAMBA_ERR_SHAPE, "tensor too large (tokens*max(2*d_inner, d_model) must be < 2^31)");
  if (io_dtype != MAMBA_F32 && io_dtype != MAMBA_BF16)
    return fail(MAMBA_ERR_DTYPE, "io_dtype must be MAMBA_F32 (0) or MAMBA_BF16 (1), got %d", io_dtype);
  return MAMBA_OK;
}

// One rocBLAS handle per thread and device.
int handle_for(hipStream_t stream, rocblas_handle* out) {
  thread_local std::vector<rocblas_handle> handles;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
    (void)hipGetLastError();
    return fail(MAMBA_ERR_DEVICE, "no HIP device is visible");
  }
  if (static_cast<size_t>(dev) >= handles.size()) handles.resize(dev + 1, nullptr);
  if (!handles[dev]) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
      (void)hipGetLastError();
      return fail(MAMBA_ERR_DEVICE, "hipGetDeviceProperties failed for device %d", dev);
    }
    if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0)
      return fail(MAMBA_ERR_DEVICE, "device %d is %s; this library is built for gfx950 only", dev, prop.gcnArchName);
    if (rocblas_create_handle(&handles[dev]) != rocblas_status_success) {
      handles[dev] = nullptr;
      return fail(MAMBA_ERR_DEVICE, "rocblas_create_handle failed on device %d", dev);
    }
  }
  if (rocblas_set_stream(handles[dev], stream) != rocblas_status_success)
    return fail(MAMBA_ERR_DEVICE, "rocblas_set_stream failed");
  *out = handles[dev];
  return MAMBA_OK;
}

// Y[m][n] = X[m][k] W[n][k]^T, all row-major in the io dtype, float32
// accumulation; X's rows are ldx elements apart (k when contiguous). In
// rocBLAS's column-major terms this is Y^T = W X^T.
int gemm(rocblas_handle h, int32_t io_dtype, int64_t m, int32_t n, int32_t k, const void* X, const void* W,
         void* Y, const char* what, int32_t ldx = 0) {
  const float one = 1.0f, zero = 0.0f;
  const rocblas_datatype t = io_dtype == MAMBA_BF16 ? rocblas_datatype_bf16_r : rocblas_datatype_f32_r;
  const rocblas_status st =
      rocblas_gemm_ex(h, rocblas_operation_transpose, rocblas_operation_none, n, static_cast<rocblas_int>(m), k,
                      &one, W, t, k, X, t, ldx ? ldx : k, &zero, Y, t, n, Y, t, n, rocblas_datatype_f32_r,
                      rocblas_gemm_algo_standard, 0, 0);
  if (st != rocblas_status_success) return fail(MAMBA_ERR_DEVICE, "%s GEMM failed: %s", what, rocblas_status_to_string(st));
  return MAMBA_OK;
}

int from_scan(int st, const char* what) {
  return fail(st, "%s: %s", what, mamba_scan_last_error());
}

// Validation shared by fwd and step. `tokens` = batch * seqlen.
int check_args(int64_t tokens, int32_t d_model, int32_t d_inner, int32_t d_state, int32_t dt_rank, int32_t io_dtype,
               const void* hidden, const void* w_in, const float* conv_w, const float* conv_b, const void* w_x,
               const void* w_dt, const float* dt_bias, const float* A, const float* D, const void* w_out,
               const void* out, void* workspace, size_t ws_need, size_t workspace_bytes) {
  const struct { const void* p; const char* n; } req[] = {
      {hidden, "hidden"}, {w_in, "w_in"}, {conv_w, "conv_w"}, {conv_b, "conv_b"}, {w_x, "w_x"}, {w_dt, "w_dt"},
      {dt_bias, "dt_bias"}, {A, "A"}, {D, "D"}, {w_out, "w_out"}, {out, "out"}};
  for (const auto& r : req)
    if (!r.p) return fail(MAMBA_ERR_NULL, "%s is NULL", r.n);
  const size_t es = io_size(io_dtype);
  for (const void* p : {hidden, w_in, w_x, w_dt, w_out, out})
    if (!aligned(p, es)) return fail(MAMBA_ERR_ALIGN, "io pointers must be %zu-byte aligned", es);
  for (const void* p : {static_cast<const void*>(conv_w), static_cast<const void*>(conv_b),
                        static_cast<const void*>(dt_bias), static_cast<const void*>(A), static_cast<const void*>(D)})
    if (!aligned(p, 4)) return fail(MAMBA_ERR_ALIGN, "float32 pointers must be 4-byte aligned");
  // out may not overlap the inputs it is computed from, nor the workspace
  const uintptr_t olo = reinterpret_cast<uintptr_t>(out), ohi = olo + static_cast<size_t>(tokens) * d_model * es;
  const struct { const void* p; size_t bytes; const char* n; } ins[] = {
      {hidden, static_cast<size_t>(tokens) * d_model * es, "hidden"},
      {w_in, 2 * static_cast<size_t>(d_inner) * d_model * es, "w_in"},
      {w_x, static_cast<size_t>(dt_rank + 2 * d_state) * d_inner * es, "w_x"},
      {w_dt, static_cast<size_t>(d_inner) * dt_rank * es, "w_dt"},
      {w_out, static_cast<size_t>(d_model) * d_inner * es, "w_out"},
      {workspace, ws_need, "workspace"}};
  for (const auto& r : ins) {
    const uintptr_t lo = reinterpret_cast<uintptr_t>(r.p), hi = lo + r.bytes;
    if (lo && lo < ohi && olo < hi) return fail(MAMBA_ERR_ALIAS, "out overlaps %s", r.n);
  }
  if (!workspace) return fail(MAMBA_ERR_WORKSPACE, "workspace is NULL but %zu bytes are required", ws_need);
  if (workspace_bytes < ws_need)
    return fail(MAMBA_ERR_WORKSPACE, "workspace has %zu bytes, %zu required", workspace_bytes, ws_need);
  if (!aligned(workspace, 256)) return fail(MAMBA_ERR_ALIGN, "workspace must be 256-byte aligned");
  return MAMBA_OK;
}

}  // namespace

extern "C" {

const char* mamba_mixer_last_error(void) { return g_last_error.c_str(); }

size_t mamba_mixer_fwd_workspace_bytes(int32_t batch, int32_t seqlen, int32_t d_model, int32_t d_inner,
                                       int32_t d_state, int32_t dt_rank, int32_t io_dtype) {
  if (batch < 1 || seqlen < 1 || d_model < 1 || d_inner < 1 || dt_rank < 1 || (d_state != 8 && d_state != 16))
    return 0;
  if (io_dtype != MAMBA_F32 && io_dtype != MAMBA_BF16) return 0;
  const int64_t tokens = static_cast<int64_t>(batch) * seqlen;
  const int64_t widest = std::max<int64_t>(std::max<int64_t>(2LL * d_inner, d_model), dt_rank + 2LL * d_state);
  if (tokens >= (int64_t{1} << 31) || tokens * widest >= (int64_t{1} << 31)) return 0;
  const size_t scan = mamba_scan_fwd_workspace_bytes(batch, seqlen, d_inner, d_state, io_dtype);
  return layout(tokens, d_inner, d_state, dt_rank, io_size(io_dtype), scan).total;
}

size_t mamba_mixer_step_workspace_bytes(int32_t batch, int32_t d_model, int32_t d_inner, int32_t d_state,
                                        int32_t dt_rank, int32_t io_dtype) {
  if (batch < 1 || d_model < 1 || d_inner < 1 || dt_rank < 1 || (d_state != 8 && d_state != 16)) return 0;
  if (io_dtype != MAMBA_F32 && io_dtype != MAMBA_BF16) return 0;
  const int64_t widest = std::max<int64_t>(std::max<int64_t>(2LL * d_inner, d_model), dt_rank + 2LL * d_state);
  if (static_cast<int64_t>(batch) * widest >= (int64_t{1} << 31)) return 0;
  return layout(batch, d_inner, d_state, dt_rank, io_size(io_dtype), 0).total;
}

int mamba_mixer_fwd(int32_t batch, int32_t seqlen, int32_t d_model, int32_t d_inner, int32_t d_state,
                    int32_t dt_rank, int32_t d_conv, int32_t io_dtype, const void* hidden, const void* w_in,
                    const float* conv_w, const float* conv_b, const void* w_x, const void* w_dt,
                    const float* dt_bias, const float* A, const float* D, const void* w_out,
                    const float* conv_state_in, const float* ssm_state_in, void* out, float* conv_state_out,
                    float* ssm_state_out, void* workspace, size_t workspace_bytes, void* stream) {
  if (batch < 1 || seqlen < 1) return fail(MAMBA_ERR_SHAPE, "batch and seqlen must be >= 1");
  const int64_t M = static_cast<int64_t>(batch) * seqlen;
  int st = check_dims(M, d_model, d_inner, d_state, dt_rank, d_conv, io_dtype);
  if (st) return st;
  const size_t es = io_size(io_dtype);
  const size_t scan_bytes = mamba_scan_fwd_workspace_bytes(batch, seqlen, d_inner, d_state, io_dtype);
  const Layout l = layout(M, d_inner, d_state, dt_rank, es, scan_bytes);
  st = check_args(M, d_model, d_inner, d_state, dt_rank, io_dtype, hidden, w_in, conv_w, conv_b, w_x, w_dt, dt_bias,
                  A, D, w_out, out, workspace, l.total, workspace_bytes);
  if (st) return st;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  rocblas_handle h;
  st = handle_for(s, &h);
  if (st) return st;
  char* ws = static_cast<char*>(workspace);
  const char* win = static_cast<const char*>(w_in);
  const char* wx = static_cast<const char*>(w_x);
  const size_t row_in = static_cast<size_t>(d_model) * es;
  // the scan with dt_proj inside serves d_state 16 and dt_rank a multiple of 8 up to 64
  const bool fused = d_state == 16 && dt_rank % 8 == 0 && dt_rank <= 64;
  // 1 in_proj as its x and z halves into contiguous arrays. (One GEMM into
  // rows (x, z), as the step does, is 19 us faster for the measured layer,
  // but the conv and the scan then read every other half-row of a buffer
  // twice as wide, which cost them 16 us more: no net gain for a sequence.)
  const int32_t xs = d_inner;  // elements between the rows of x and of z
  const char* zp = ws + l.z;
  if ((st = gemm(h, io_dtype, M, d_inner, d_model, hidden, win, ws + l.x, "in_proj (x)"))) return st;
  if ((st = gemm(h, io_dtype, M, d_inner, d_model, hidden, win + d_inner * row_in, ws + l.z, "in_proj (z)")))
    return st;
  // 2 conv + SiLU feeding x_proj and the scan; then the conv state (after the
  // conv kernel has read the history, so the state may be updated in place)
  hipError_t e = mmix::launch_conv_silu(io_dtype, batch, seqlen, d_inner, ws + l.x, xs, conv_w, conv_b,
                                        conv_state_in, ws + l.xc, s);
  if (e == hipSuccess)
    e = mmix::launch_conv_state(io_dtype, batch, seqlen, d_inner, ws + l.x, xs, conv_state_in, conv_state_out, s);
  if (e != hipSuccess) return fail(MAMBA_ERR_DEVICE, "conv kernel launch failed: %s", hipGetErrorString(e));
  // 3 x_proj: dt_low, B and C of a token side by side in one row
  const int32_t xw = dt_rank + 2 * d_state;
  if ((st = gemm(h, io_dtype, M, xw, d_inner, ws + l.xc, wx, ws + l.xp, "x_proj"))) return st;
  const char* Bp = ws + l.xp + dt_rank * es;
  if (fused) {
    // 4-6 dt_proj on the matrix cores inside the scan (dt is never stored),
    // softplus, scan and gate from the stored xc; dt_low, B, C and z in place
    st = mamba_scan_fwd_xc_dtproj(batch, seqlen, d_inner, d_state, dt_rank, io_dtype, ws + l.xc, ws + l.xp, xw, w_dt,
                                  zp, xs, Bp, Bp + d_state * es, xw, dt_bias, D, A, ssm_state_in, ws + l.y,
                                  ssm_state_out, scan_bytes ? ws + l.scan : nullptr, scan_bytes, stream);
  } else {
    // 4 dt_proj from dt_low in place (its bias is applied inside the scan's softplus)
    if ((st = gemm(h, io_dtype, M, d_inner, dt_rank, ws + l.xp, w_dt, ws + l.dt, "dt_proj", xw))) return st;
    // 5-6 selective scan with gate, from the stored xc (no second conv), B and C in place
    st = mamba_scan_fwd_xc(batch, seqlen, d_inner, d_state, io_dtype, ws + l.xc, ws + l.dt, ws + l.z, Bp,
                           Bp + d_state * es, xw, dt_bias, D, A, ssm_state_in, ws + l.y, ssm_state_out,
                           scan_bytes ? ws + l.scan : nullptr, scan_bytes, stream);
  }
  if (st) return from_scan(st, "selective scan");
  // 7 out_proj
  if ((st = gemm(h, io_dtype, M, d_model, d_inner, ws + l.y, w_out, out, "out_proj"))) return st;
  return ok();
}

int mamba_mixer_step(int32_t batch, int32_t d_model, int32_t d_inner, int32_t d_state, int32_t dt_rank,
                     int32_t d_conv, int32_t io_dtype, const void* hidden, const void* w_in, const float* conv_w,
                     const float* conv_b, const void* w_x, const void* w_dt, const float* dt_bias, const float* A,
                     const float* D, const void* w_out, const float* conv_state_in, const float* ssm_state_in,
                     void* out, float* conv_state_out, float* ssm_state_out, void* workspace,
                     size_t workspace_bytes, void* stream) {
  if (batch < 1) return fail(MAMBA_ERR_SHAPE, "batch must be >= 1");
  const int64_t M = batch;
  int st = check_dims(M, d_model, d_inner, d_state, dt_rank, d_conv, io_dtype);
  if (st) return st;
  if (!conv_state_in || !ssm_state_in || !conv_state_out || !ssm_state_out)
    return fail(MAMBA_ERR_NULL, "the step needs all four state pointers");
  const size_t es = io_size(io_dtype);
  const Layout l = layout(M, d_inner, d_state, dt_rank, es, 0);
  st = check_args(M, d_model, d_inner, d_state, dt_rank, io_dtype, hidden, w_in, conv_w, conv_b, w_x, w_dt, dt_bias,
                  A, D, w_out, out, workspace, l.total, workspace_bytes);
  if (st) return st;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  rocblas_handle h;
  st = handle_for(s, &h);
  if (st) return st;
  char* ws = static_cast<char*>(workspace);
  const char* win = static_cast<const char*>(w_in);
  const char* wx = static_cast<const char*>(w_x);
  // in_proj as one GEMM: row b holds the token's x, then its z
  if ((st = gemm(h, io_dtype, M, 2 * d_inner, d_model, hidden, win, ws + l.x, "in_proj"))) return st;
  const int32_t xs = 2 * d_inner;
  // xc of the token from the incoming conv state, and the new conv state
  hipError_t e = mmix::launch_conv_silu_step(io_dtype, batch, d_inner, ws + l.x, xs, conv_w, conv_b, conv_state_in,
                                             ws + l.xc, conv_state_out, s);
  if (e != hipSuccess) return fail(MAMBA_ERR_DEVICE, "conv kernel launch failed: %s", hipGetErrorString(e));
  const int32_t xw = dt_rank + 2 * d_state;
  if ((st = gemm(h, io_dtype, M, xw, d_inner, ws + l.xc, wx, ws + l.xp, "x_proj"))) return st;
  // dt_proj, softplus, scan, readout and gate in one kernel: dt_low, B and C read in place
  const char* Bp = ws + l.xp + dt_rank * es;
  st = mamba_scan_step_xc_dtproj(batch, d_inner, d_state, dt_rank, io_dtype, ws + l.xc, ws + l.xp, xw, w_dt,
                                 ws + l.x + d_inner * es, xs, Bp, Bp + d_state * es, xw, dt_bias, D, A, ssm_state_in,
                                 ws + l.y, ssm_state_out, stream);
  if (st) return from_scan(st, "selective scan step");
  if ((st = gemm(h, io_dtype, M, d_model, d_inner, ws + l.y, w_out, out, "out_proj"))) return st;
  return ok();
}

}  // extern "C"
