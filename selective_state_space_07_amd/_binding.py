"""ctypes binding of libmamba_scan.so (declared in include/mamba_scan.h).

Argument marshalling only: device pointers of torch tensors, the current HIP
stream, and status codes turned into exceptions. Every step of the scan runs
in the library's HIP kernels; nothing here computes the method.
"""
import ctypes
import os

from . import build as _build

MAMBA_F32 = 0
MAMBA_BF16 = 1
STATUS = {0: "MAMBA_OK", 1: "MAMBA_ERR_NULL", 2: "MAMBA_ERR_SHAPE", 3: "MAMBA_ERR_DTYPE",
          4: "MAMBA_ERR_ALIGN", 5: "MAMBA_ERR_ALIAS", 6: "MAMBA_ERR_WORKSPACE", 7: "MAMBA_ERR_DEVICE"}

# Every symbol include/mamba_scan.h declares.
EXPORTS = ("mamba_scan_abi_version", "mamba_scan_status_str", "mamba_scan_last_error",
           "mamba_scan_call_count", "mamba_scan_fwd_workspace_bytes", "mamba_scan_fwd", "mamba_scan_fwd_seq",
           "mamba_scan_ckpt_bytes", "mamba_scan_fwd_ckpt", "mamba_scan_bwd_workspace_bytes", "mamba_scan_bwd",
           "mamba_scan_bwd_ckpt_workspace_bytes", "mamba_scan_bwd_ckpt", "mamba_scan_step", "mamba2_ssd_fwd_workspace_bytes",
           "mamba2_ssd_fwd", "mamba2_ssd_fwd_seq", "mamba2_ssd_step", "mamba_scan_fwd_noalloc", "mamba_scan_fwd_xc",
           "mamba_scan_step_xc", "mamba_scan_step_xc_dtproj", "mamba_scan_fwd_xc_dtproj")
NOALLOC_SCRATCH_BYTES = 8 << 20  # MAMBA_SCAN_NOALLOC_SCRATCH_BYTES
# Every symbol include/mamba_scan_testing.h declares (test suites only).
TESTING_EXPORTS = ("mamba_scan_testing_fwd_workspace_bytes", "mamba_scan_testing_fwd")


class MambaScanError(RuntimeError):
    """A libmamba_scan call returned a non-zero status."""

    def __init__(self, status, message):
        super().__init__(message)
        self.status = status


_lib = None


def library_path():
    return _build.LIB


def load():
    """Load libmamba_scan.so (building it first if it is absent) and declare signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_build.LIB):
        _build.build()
    lib = ctypes.CDLL(_build.LIB)
    i32, vp, sz = ctypes.c_int32, ctypes.c_void_p, ctypes.c_size_t
    lib.mamba_scan_abi_version.restype = ctypes.c_int
    lib.mamba_scan_abi_version.argtypes = []
    lib.mamba_scan_status_str.restype = ctypes.c_char_p
    lib.mamba_scan_status_str.argtypes = [ctypes.c_int]
    lib.mamba_scan_last_error.restype = ctypes.c_char_p
    lib.mamba_scan_last_error.argtypes = []
    lib.mamba_scan_call_count.restype = ctypes.c_uint64
    lib.mamba_scan_call_count.argtypes = []
    lib.mamba_scan_fwd_workspace_bytes.restype = sz
    lib.mamba_scan_fwd_workspace_bytes.argtypes = [i32] * 5
    lib.mamba_scan_fwd.restype = ctypes.c_int
    lib.mamba_scan_fwd.argtypes = [i32] * 6 + [vp] * 16 + [sz, vp]
    lib.mamba_scan_fwd_seq.restype = ctypes.c_int
    lib.mamba_scan_fwd_seq.argtypes = [i32] * 6 + [vp] * 17 + [sz, vp]
    lib.mamba_scan_ckpt_bytes.restype = sz
    lib.mamba_scan_ckpt_bytes.argtypes = [i32] * 4
    lib.mamba_scan_fwd_ckpt.restype = ctypes.c_int
    lib.mamba_scan_fwd_ckpt.argtypes = [i32] * 6 + [vp] * 17 + [sz, vp]
    lib.mamba_scan_bwd_ckpt_workspace_bytes.restype = sz
    lib.mamba_scan_bwd_ckpt_workspace_bytes.argtypes = [i32] * 5
    lib.mamba_scan_bwd_ckpt.restype = ctypes.c_int
    lib.mamba_scan_bwd_ckpt.argtypes = [i32] * 6 + [vp] * 24 + [vp, sz, vp]
    lib.mamba_scan_bwd_workspace_bytes.restype = sz
    lib.mamba_scan_bwd_workspace_bytes.argtypes = [i32] * 5
    lib.mamba_scan_bwd.restype = ctypes.c_int
    lib.mamba_scan_bwd.argtypes = [i32] * 6 + [vp] * 23 + [vp, sz, vp]
    lib.mamba2_ssd_fwd_workspace_bytes.restype = sz
    lib.mamba2_ssd_fwd_workspace_bytes.argtypes = [i32] * 7
    lib.mamba2_ssd_fwd.restype = ctypes.c_int
    lib.mamba2_ssd_fwd.argtypes = [i32] * 7 + [vp] * 10 + [vp, sz, vp]
    lib.mamba2_ssd_fwd_seq.restype = ctypes.c_int
    lib.mamba2_ssd_fwd_seq.argtypes = [i32] * 7 + [vp] * 11 + [vp, sz, vp]
    lib.mamba2_ssd_step.restype = ctypes.c_int
    lib.mamba2_ssd_step.argtypes = [i32] * 6 + [vp] * 10 + [vp]
    lib.mamba_scan_step.restype = ctypes.c_int
    lib.mamba_scan_step.argtypes = [i32] * 5 + [vp] * 15 + [vp]
    lib.mamba_scan_fwd_xc.restype = ctypes.c_int
    lib.mamba_scan_fwd_xc.argtypes = [i32] * 5 + [vp] * 5 + [i32] + [vp] * 6 + [vp, sz, vp]
    lib.mamba_scan_fwd_xc_dtproj.restype = ctypes.c_int
    lib.mamba_scan_fwd_xc_dtproj.argtypes = ([i32] * 6 + [vp, vp, i32, vp, vp, i32, vp, vp, i32] + [vp] * 6
                                             + [vp, sz, vp])
    lib.mamba_scan_step_xc.restype = ctypes.c_int
    lib.mamba_scan_step_xc.argtypes = [i32] * 4 + [vp] * 5 + [i32] + [vp] * 6 + [vp]
    lib.mamba_scan_step_xc_dtproj.restype = ctypes.c_int
    lib.mamba_scan_step_xc_dtproj.argtypes = ([i32] * 5 + [vp, vp, i32, vp, vp, i32, vp, vp, i32] + [vp] * 6
                                              + [vp])
    lib.mamba_scan_fwd_noalloc.restype = ctypes.c_int
    lib.mamba_scan_fwd_noalloc.argtypes = [i32] * 6 + [vp] * 15 + [vp]
    lib.mamba_scan_testing_fwd_workspace_bytes.restype = sz
    lib.mamba_scan_testing_fwd_workspace_bytes.argtypes = [i32] * 6
    lib.mamba_scan_testing_fwd.restype = ctypes.c_int
    lib.mamba_scan_testing_fwd.argtypes = [i32] * 8 + [vp] * 18 + [sz, vp]
    _lib = lib
    return lib


def _check(lib, status, what):
    if status != 0:
        detail = lib.mamba_scan_last_error().decode(errors="replace")
        raise MambaScanError(status, "%s failed: %s" % (what, detail or STATUS.get(status, status)))


def mamba_scan_abi_version():
    return load().mamba_scan_abi_version()


def mamba_scan_status_str(status):
    return load().mamba_scan_status_str(int(status)).decode()


def mamba_scan_last_error():
    return load().mamba_scan_last_error().decode(errors="replace")


def mamba_scan_call_count():
    return int(load().mamba_scan_call_count())


def mamba_scan_fwd_workspace_bytes(batch, seqlen, d_inner, d_state, io_dtype):
    return int(load().mamba_scan_fwd_workspace_bytes(batch, seqlen, d_inner, d_state, io_dtype))


def mamba_scan_fwd(batch, seqlen, d_inner, d_state, d_conv, io_dtype, x, dt, z, B, C, conv_w, conv_b,
                   dt_bias, D, A, conv_state_in, ssm_state_in, y, conv_state_out, ssm_state_out, workspace,
                   workspace_bytes, stream, check=True):
    """Raw call with integer device addresses (0 for NULL). Returns the status;
    raises MambaScanError on a non-zero status when `check` is true."""
    lib = load()
    st = lib.mamba_scan_fwd(batch, seqlen, d_inner, d_state, d_conv, io_dtype, x, dt, z, B, C, conv_w, conv_b,
                            dt_bias, D, A, conv_state_in, ssm_state_in, y, conv_state_out, ssm_state_out,
                            workspace, workspace_bytes, stream)
    if check:
        _check(lib, st, "mamba_scan_fwd")
    return st


def mamba_scan_fwd_seq(batch, seqlen, d_inner, d_state, d_conv, io_dtype, x, dt, z, B, C, seq_idx, conv_w,
                       conv_b, dt_bias, D, A, conv_state_in, ssm_state_in, y, conv_state_out, ssm_state_out,
                       workspace, workspace_bytes, stream, check=True):
    """Raw call with integer device addresses (0 for NULL); seq_idx is an int32
    [batch][seqlen] device array of document ids; see mamba_scan_fwd."""
    lib = load()
    st = lib.mamba_scan_fwd_seq(batch, seqlen, d_inner, d_state, d_conv, io_dtype, x, dt, z, B, C, seq_idx,
                                conv_w, conv_b, dt_bias, D, A, conv_state_in, ssm_state_in, y, conv_state_out,
                                ssm_state_out, workspace, workspace_bytes, stream)
    if check:
        _check(lib, st, "mamba_scan_fwd_seq")
    return st


def mamba_scan_ckpt_bytes(batch, seqlen, d_inner, d_state):
    return int(load().mamba_scan_ckpt_bytes(batch, seqlen, d_inner, d_state))


def mamba_scan_fwd_ckpt(batch, seqlen, d_inner, d_state, d_conv, io_dtype, x, dt, z, B, C, conv_w, conv_b,
                        dt_bias, D, A, conv_state_in, ssm_state_in, y, conv_state_out, ssm_state_out, ckpt,
                        workspace, workspace_bytes, stream, check=True):
    """Raw call with integer device addresses (0 for NULL); see mamba_scan_fwd."""
    lib = load()
    st = lib.mamba_scan_fwd_ckpt(batch, seqlen, d_inner, d_state, d_conv, io_dtype, x, dt, z, B, C, conv_w, conv_b,
                                 dt_bias, D, A, conv_state_in, ssm_state_in, y, conv_state_out, ssm_state_out, ckpt,
                                 workspace, workspace_bytes, stream)
    if check:
        _check(lib, st, "mamba_scan_fwd_ckpt")
    return st


def mamba_scan_bwd_ckpt_workspace_bytes(batch, seqlen, d_inner, d_state, io_dtype):
    return int(load().mamba_scan_bwd_ckpt_workspace_bytes(batch, seqlen, d_inner, d_state, io_dtype))


def mamba_scan_bwd_ckpt(batch, seqlen, d_inner, d_state, d_conv, io_dtype, x, dt, z, B, C, conv_w, conv_b, dt_bias,
                        D, A, conv_state_in, ssm_state_in, dy, dx, ddt, dz, dB, dC, dconv_w, dconv_b, ddt_bias, dD,
                        dA, ckpt, workspace, workspace_bytes, stream, check=True):
    """Raw call with integer device addresses (0 for NULL); see mamba_scan_bwd."""
    lib = load()
    st = lib.mamba_scan_bwd_ckpt(batch, seqlen, d_inner, d_state, d_conv, io_dtype, x, dt, z, B, C, conv_w, conv_b,
                                 dt_bias, D, A, conv_state_in, ssm_state_in, dy, dx, ddt, dz, dB, dC, dconv_w,
                                 dconv_b, ddt_bias, dD, dA, ckpt, workspace, workspace_bytes, stream)
    if check:
        _check(lib, st, "mamba_scan_bwd_ckpt")
    return st


def mamba_scan_bwd_workspace_bytes(batch, seqlen, d_inner, d_state, io_dtype):
    return int(load().mamba_scan_bwd_workspace_bytes(batch, seqlen, d_inner, d_state, io_dtype))


def mamba_scan_bwd(batch, seqlen, d_inner, d_state, d_conv, io_dtype, x, dt, z, B, C, conv_w, conv_b, dt_bias, D,
                   A, conv_state_in, ssm_state_in, dy, dx, ddt, dz, dB, dC, dconv_w, dconv_b, ddt_bias, dD, dA,
                   workspace, workspace_bytes, stream, check=True):
    """Raw call with integer device addresses (0 for NULL); see mamba_scan_fwd."""
    lib = load()
    st = lib.mamba_scan_bwd(batch, seqlen, d_inner, d_state, d_conv, io_dtype, x, dt, z, B, C, conv_w, conv_b,
                            dt_bias, D, A, conv_state_in, ssm_state_in, dy, dx, ddt, dz, dB, dC, dconv_w, dconv_b,
                            ddt_bias, dD, dA, workspace, workspace_bytes, stream)
    if check:
        _check(lib, st, "mamba_scan_bwd")
    return st


def mamba2_ssd_fwd_workspace_bytes(batch, seqlen, nheads, headdim, d_state, ngroups, io_dtype):
    return int(load().mamba2_ssd_fwd_workspace_bytes(batch, seqlen, nheads, headdim, d_state, ngroups, io_dtype))


def mamba2_ssd_fwd(batch, seqlen, nheads, headdim, d_state, ngroups, io_dtype, x, dt, B, C, dt_bias, A, D, state_in,
                   y, state_out, workspace, workspace_bytes, stream, check=True):
    """Raw call with integer device addresses (0 for NULL); see include/mamba2_ssd.h."""
    lib = load()
    st = lib.mamba2_ssd_fwd(batch, seqlen, nheads, headdim, d_state, ngroups, io_dtype, x, dt, B, C, dt_bias, A, D,
                            state_in, y, state_out, workspace, workspace_bytes, stream)
    if check:
        _check(lib, st, "mamba2_ssd_fwd")
    return st


def mamba2_ssd_fwd_seq(batch, seqlen, nheads, headdim, d_state, ngroups, io_dtype, x, dt, B, C, seq_idx, dt_bias, A,
                       D, state_in, y, state_out, workspace, workspace_bytes, stream, check=True):
    """Raw call with integer device addresses (0 for NULL); see include/mamba2_ssd.h."""
    lib = load()
    st = lib.mamba2_ssd_fwd_seq(batch, seqlen, nheads, headdim, d_state, ngroups, io_dtype, x, dt, B, C, seq_idx,
                                dt_bias, A, D, state_in, y, state_out, workspace, workspace_bytes, stream)
    if check:
        _check(lib, st, "mamba2_ssd_fwd_seq")
    return st


def mamba2_ssd_step(batch, nheads, headdim, d_state, ngroups, io_dtype, x, dt, B, C, dt_bias, A, D, state_in, y,
                    state_out, stream, check=True):
    """Raw call with integer device addresses; see include/mamba2_ssd.h."""
    lib = load()
    st = lib.mamba2_ssd_step(batch, nheads, headdim, d_state, ngroups, io_dtype, x, dt, B, C, dt_bias, A, D, state_in,
                             y, state_out, stream)
    if check:
        _check(lib, st, "mamba2_ssd_step")
    return st


def mamba_scan_step(batch, d_inner, d_state, d_conv, io_dtype, x, dt, z, B, C, conv_w, conv_b, dt_bias, D, A,
                    conv_state_in, ssm_state_in, y, conv_state_out, ssm_state_out, stream, check=True):
    """Raw call with integer device addresses (0 for NULL); see mamba_scan_fwd."""
    lib = load()
    st = lib.mamba_scan_step(batch, d_inner, d_state, d_conv, io_dtype, x, dt, z, B, C, conv_w, conv_b, dt_bias,
                             D, A, conv_state_in, ssm_state_in, y, conv_state_out, ssm_state_out, stream)
    if check:
        _check(lib, st, "mamba_scan_step")
    return st


def mamba_scan_testing_fwd_workspace_bytes(kind, batch, seqlen, d_inner, d_state, io_dtype):
    return load().mamba_scan_testing_fwd_workspace_bytes(kind, batch, seqlen, d_inner, d_state, io_dtype)


def mamba_scan_testing_fwd(kind, force_wide, batch, seqlen, d_inner, d_state, d_conv, io_dtype, x, dt, z, B, C,
                           seq_idx, conv_w, conv_b, dt_bias, D, A, conv_state_in, ssm_state_in, y, conv_state_out,
                           ssm_state_out, ckpt, workspace, workspace_bytes, stream, check=True):
    """Raw call of the testing entry point (include/mamba_scan_testing.h), as mamba_scan_fwd."""
    lib = load()
    st = lib.mamba_scan_testing_fwd(kind, force_wide, batch, seqlen, d_inner, d_state, d_conv, io_dtype, x, dt, z, B,
                                    C, seq_idx, conv_w, conv_b, dt_bias, D, A, conv_state_in, ssm_state_in, y,
                                    conv_state_out, ssm_state_out, ckpt, workspace, workspace_bytes, stream)
    if check:
        _check(lib, st, "mamba_scan_testing_fwd")
    return st


def mamba_scan_fwd_noalloc(batch, seqlen, d_inner, d_state, d_conv, io_dtype, x, dt, z, B, C, conv_w, conv_b,
                           dt_bias, D, A, conv_state_in, ssm_state_in, y, conv_state_out, ssm_state_out, stream,
                           check=True):
    """Raw call of the prefill that takes its workspace from the library's
    fixed device scratch (include/mamba_scan.h, mamba_scan_fwd_noalloc)."""
    lib = load()
    st = lib.mamba_scan_fwd_noalloc(batch, seqlen, d_inner, d_state, d_conv, io_dtype, x, dt, z, B, C, conv_w,
                                    conv_b, dt_bias, D, A, conv_state_in, ssm_state_in, y, conv_state_out,
                                    ssm_state_out, stream)
    if check:
        _check(lib, st, "mamba_scan_fwd_noalloc")
    return st


def mamba_scan_fwd_xc(batch, seqlen, d_inner, d_state, io_dtype, xc, dt, z, B, C, bc_stride, dt_bias, D, A,
                      ssm_state_in, y, ssm_state_out, workspace, workspace_bytes, stream, check=True):
    """Raw call of the prefill from the activated conv output xc (no conv
    inside); the rows of B and C are bc_stride elements apart."""
    lib = load()
    st = lib.mamba_scan_fwd_xc(batch, seqlen, d_inner, d_state, io_dtype, xc, dt, z, B, C, bc_stride, dt_bias, D, A,
                               ssm_state_in, y, ssm_state_out, workspace, workspace_bytes, stream)
    if check:
        _check(lib, st, "mamba_scan_fwd_xc")
    return st


def mamba_scan_fwd_xc_dtproj(batch, seqlen, d_inner, d_state, dt_rank, io_dtype, xc, dt_low, dtl_stride, w_dt, z,
                             z_stride, B, C, bc_stride, dt_bias, D, A, ssm_state_in, y, ssm_state_out, workspace,
                             workspace_bytes, stream, check=True):
    """Raw call of the prefill from xc with dt = dt_low . w_dt[d] computed
    inside (on the matrix cores); the rows of z are z_stride elements apart."""
    lib = load()
    st = lib.mamba_scan_fwd_xc_dtproj(batch, seqlen, d_inner, d_state, dt_rank, io_dtype, xc, dt_low, dtl_stride, w_dt,
                                      z, z_stride, B, C, bc_stride, dt_bias, D, A, ssm_state_in, y, ssm_state_out,
                                      workspace, workspace_bytes, stream)
    if check:
        _check(lib, st, "mamba_scan_fwd_xc_dtproj")
    return st


def mamba_scan_step_xc(batch, d_inner, d_state, io_dtype, xc, dt, z, B, C, bc_stride, dt_bias, D, A, ssm_state_in,
                       y, ssm_state_out, stream, check=True):
    """Raw call of one token from its activated conv output xc (no conv, no
    conv states); the batch rows of B and C are bc_stride elements apart."""
    lib = load()
    st = lib.mamba_scan_step_xc(batch, d_inner, d_state, io_dtype, xc, dt, z, B, C, bc_stride, dt_bias, D, A,
                                ssm_state_in, y, ssm_state_out, stream)
    if check:
        _check(lib, st, "mamba_scan_step_xc")
    return st


def mamba_scan_step_xc_dtproj(batch, d_inner, d_state, dt_rank, io_dtype, xc, dt_low, dtl_stride, w_dt, z, z_stride,
                              B, C, bc_stride, dt_bias, D, A, ssm_state_in, y, ssm_state_out, stream, check=True):
    """Raw call of one token from xc with dt = dt_low . w_dt[d] computed
    inside; the batch rows of z are z_stride elements apart."""
    lib = load()
    st = lib.mamba_scan_step_xc_dtproj(batch, d_inner, d_state, dt_rank, io_dtype, xc, dt_low, dtl_stride, w_dt, z,
                                       z_stride, B, C, bc_stride, dt_bias, D, A, ssm_state_in, y, ssm_state_out,
                                       stream)
    if check:
        _check(lib, st, "mamba_scan_step_xc_dtproj")
    return st
