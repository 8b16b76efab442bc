"""ctypes binding and torch-facing API of libmamba_mixer.so (declared in
include/mamba_mixer.h): one Mamba-1 mixer layer (in_proj, conv + SiLU,
x_proj, dt_proj + softplus, selective scan, gate, out_proj) on the GPU.

Argument marshalling only: the projections run as rocBLAS GEMMs and every
other step in the HIP kernels of libmamba_mixer / libmamba_scan.
"""
import ctypes
import os
from dataclasses import dataclass

import torch

from . import _binding as _b
from . import build as _build
from .api import check_out, check_workspace

EXPORTS = ("mamba_mixer_last_error", "mamba_mixer_fwd_workspace_bytes", "mamba_mixer_fwd",
           "mamba_mixer_step_workspace_bytes", "mamba_mixer_step")
_IO = {torch.float32: _b.MAMBA_F32, torch.bfloat16: _b.MAMBA_BF16}
_lib = None


def load():
    """Load libmamba_mixer.so (building it and the scan library if absent)."""
    global _lib
    if _lib is not None:
        return _lib
    _b.load()  # the scan library it links against
    if not os.path.exists(_build.MIXER_LIB):
        _build.build_mixer()
    lib = ctypes.CDLL(_build.MIXER_LIB)
    i32, vp, sz = ctypes.c_int32, ctypes.c_void_p, ctypes.c_size_t
    lib.mamba_mixer_last_error.restype = ctypes.c_char_p
    lib.mamba_mixer_last_error.argtypes = []
    lib.mamba_mixer_fwd_workspace_bytes.restype = sz
    lib.mamba_mixer_fwd_workspace_bytes.argtypes = [i32] * 7
    lib.mamba_mixer_step_workspace_bytes.restype = sz
    lib.mamba_mixer_step_workspace_bytes.argtypes = [i32] * 6
    lib.mamba_mixer_fwd.restype = ctypes.c_int
    lib.mamba_mixer_fwd.argtypes = [i32] * 8 + [vp] * 15 + [vp, sz, vp]
    lib.mamba_mixer_step.restype = ctypes.c_int
    lib.mamba_mixer_step.argtypes = [i32] * 7 + [vp] * 15 + [vp, sz, vp]
    _lib = lib
    return lib


def library_path():
    return _build.MIXER_LIB


@dataclass
class MixerWeights:
    """One layer's parameters: w_in [2*d_inner, d_model], w_x [dt_rank + 2*d_state, d_inner],
    w_dt [d_inner, dt_rank], w_out [d_model, d_inner] in the io dtype; conv_w [d_inner, 4],
    conv_b, dt_bias, D [d_inner], A [d_inner, d_state] in float32."""
    w_in: torch.Tensor
    conv_w: torch.Tensor
    conv_b: torch.Tensor
    w_x: torch.Tensor
    w_dt: torch.Tensor
    dt_bias: torch.Tensor
    A: torch.Tensor
    D: torch.Tensor
    w_out: torch.Tensor

    def dims(self):
        d2, d_model = self.w_in.shape
        d_inner = d2 // 2
        dt_rank = self.w_dt.shape[1]
        d_state = (self.w_x.shape[0] - dt_rank) // 2
        return d_model, d_inner, d_state, dt_rank


def _check(lib, st, what):
    if st != 0:
        raise _b.MambaScanError(st, "%s failed: %s" % (what, lib.mamba_mixer_last_error().decode(errors="replace")))


def _prep(w, hidden):
    io = hidden.dtype
    if io not in _IO:
        raise TypeError("hidden must be float32 or bfloat16 (got %s)" % io)
    out = []
    for name in ("w_in", "conv_w", "conv_b", "w_x", "w_dt", "dt_bias", "A", "D", "w_out"):
        t = getattr(w, name)
        want = io if name in ("w_in", "w_x", "w_dt", "w_out") else torch.float32
        if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
            raise _b.MambaScanError(7, "%s must be a GPU tensor; there is no CPU path" % name)
        if t.dtype != want:
            raise TypeError("%s must be %s (got %s)" % (name, want, t.dtype))
        out.append(t.contiguous())
    return out


def _state(t, shape, name):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda" or t.dtype != torch.float32:
        raise _b.MambaScanError(7, "%s must be a float32 GPU tensor" % name)
    if tuple(t.shape) != tuple(shape):
        raise _b.MambaScanError(2, "%s must be %s (got %s)" % (name, tuple(shape), tuple(t.shape)))
    return t.contiguous()


def workspace_bytes(batch, seqlen, d_model, d_inner, d_state, dt_rank, dtype):
    return int(load().mamba_mixer_fwd_workspace_bytes(batch, seqlen, d_model, d_inner, d_state, dt_rank, _IO[dtype]))


def step_workspace_bytes(batch, d_model, d_inner, d_state, dt_rank, dtype):
    return int(load().mamba_mixer_step_workspace_bytes(batch, d_model, d_inner, d_state, dt_rank, _IO[dtype]))


def _ws(nbytes, device, workspace):
    if workspace is not None:
        return workspace
    return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)


def mixer_fwd(hidden, w, conv_state=None, ssm_state=None, *, out=None, workspace=None):
    """hidden [batch, seqlen, d_model] -> (out [batch, seqlen, d_model], conv_state', ssm_state')."""
    lib = load()
    if hidden.device.type != "cuda":
        raise _b.MambaScanError(7, "hidden must be on the GPU; there is no CPU path")
    hidden = hidden.contiguous()
    w_in, conv_w, conv_b, w_x, w_dt, dt_bias, A, D, w_out = _prep(w, hidden)
    batch, seqlen, d_model = hidden.shape
    _, d_inner, d_state, dt_rank = w.dims()
    io = _IO[hidden.dtype]
    f32 = torch.float32
    conv_state = _state(conv_state, (batch, d_inner, 3), "conv_state")
    ssm_state = _state(ssm_state, (batch, d_inner, d_state), "ssm_state")
    if out is not None:
        check_out(out, "out", (batch, seqlen, d_model), hidden.dtype, hidden.device)
    else:
        out = torch.empty(batch, seqlen, d_model, dtype=hidden.dtype, device=hidden.device)
    workspace = check_workspace(workspace, hidden.device)
    cso = torch.empty(batch, d_inner, 3, dtype=f32, device=hidden.device)
    sso = torch.empty(batch, d_inner, d_state, dtype=f32, device=hidden.device)
    need = lib.mamba_mixer_fwd_workspace_bytes(batch, seqlen, d_model, d_inner, d_state, dt_rank, io)
    ws = _ws(need, hidden.device, workspace)
    a = lambda t: 0 if t is None else t.contiguous().data_ptr()
    st = lib.mamba_mixer_fwd(batch, seqlen, d_model, d_inner, d_state, dt_rank, 4, io, a(hidden), a(w_in), a(conv_w),
                             a(conv_b), a(w_x), a(w_dt), a(dt_bias), a(A), a(D), a(w_out), a(conv_state),
                             a(ssm_state), a(out), a(cso), a(sso), a(ws), ws.numel() * ws.element_size(),
                             torch.cuda.current_stream(hidden.device).cuda_stream)
    _check(lib, st, "mamba_mixer_fwd")
    return out, cso, sso


def mixer_step(hidden, w, conv_state, ssm_state, *, inplace=False, out=None, workspace=None):
    """hidden [batch, d_model] -> (out [batch, d_model], conv_state', ssm_state'); states required."""
    lib = load()
    if hidden.device.type != "cuda":
        raise _b.MambaScanError(7, "hidden must be on the GPU; there is no CPU path")
    hidden = hidden.contiguous()
    w_in, conv_w, conv_b, w_x, w_dt, dt_bias, A, D, w_out = _prep(w, hidden)
    batch, d_model = hidden.shape
    _, d_inner, d_state, dt_rank = w.dims()
    io = _IO[hidden.dtype]
    if conv_state is None or ssm_state is None:
        raise _b.MambaScanError(1, "the step needs conv_state and ssm_state")
    if inplace and not (conv_state.is_contiguous() and ssm_state.is_contiguous()):
        raise _b.MambaScanError(2, "in-place step needs contiguous state tensors")
    conv_state = _state(conv_state, (batch, d_inner, 3), "conv_state")
    ssm_state = _state(ssm_state, (batch, d_inner, d_state), "ssm_state")
    if out is not None:
        check_out(out, "out", (batch, d_model), hidden.dtype, hidden.device)
    else:
        out = torch.empty(batch, d_model, dtype=hidden.dtype, device=hidden.device)
    workspace = check_workspace(workspace, hidden.device)
    if inplace:
        cso, sso = conv_state, ssm_state
    else:
        cso, sso = torch.empty_like(conv_state), torch.empty_like(ssm_state)
    need = lib.mamba_mixer_step_workspace_bytes(batch, d_model, d_inner, d_state, dt_rank, io)
    ws = _ws(need, hidden.device, workspace)
    a = lambda t: t.data_ptr()
    st = lib.mamba_mixer_step(batch, d_model, d_inner, d_state, dt_rank, 4, io, a(hidden), a(w_in), a(conv_w),
                              a(conv_b), a(w_x), a(w_dt), a(dt_bias), a(A), a(D), a(w_out), a(conv_state),
                              a(ssm_state), a(out), a(cso), a(sso), a(ws), ws.numel() * ws.element_size(),
                              torch.cuda.current_stream(hidden.device).cuda_stream)
    _check(lib, st, "mamba_mixer_step")
    return out, cso, sso
