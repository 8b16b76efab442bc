"""torch-tensor front end of libmamba_scan: `fwd` (prefill, optionally writing
checkpoints for the backward), `bwd` (its gradients) and `step` (decode).

Marshalling only: checks that tensors are CUDA (HIP) tensors of the declared
dtypes, makes them contiguous, allocates outputs and the workspace, and passes
raw device addresses plus torch's current HIP stream to the C ABI. The
arithmetic is all in the library's kernels.
"""
from dataclasses import dataclass

import torch

from . import _binding as _b

_IO = {torch.float32: _b.MAMBA_F32, torch.bfloat16: _b.MAMBA_BF16}


@dataclass
class Params:
    """Per-channel parameters of one mixer layer, all float32 on the GPU.

    conv_w [d_inner, 4] (tap 3 multiplies the newest token), conv_b [d_inner],
    dt_bias [d_inner], D [d_inner], A [d_inner, d_state] (A = -exp(A_log)).
    """
    conv_w: torch.Tensor
    conv_b: torch.Tensor
    dt_bias: torch.Tensor
    D: torch.Tensor
    A: torch.Tensor

    def to(self, device):
        return Params(*(t.to(device) for t in (self.conv_w, self.conv_b, self.dt_bias, self.D, self.A)))


def _addr(t):
    return 0 if t is None else t.data_ptr()


def _dev(t, name, dtype=None):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.device.type != "cuda":
        raise _b.MambaScanError(7, "%s must be on the GPU (got %s); there is no CPU path" % (name, t.device))
    if dtype is not None and t.dtype != dtype:
        raise TypeError("%s must be %s (got %s)" % (name, dtype, t.dtype))
    return t.contiguous()


def check_out(t, name, shape, dtype, device):
    """A caller-supplied output (or checkpoint) tensor must be exactly what the
    kernels write: the shape, dtype and device given, and contiguous (the
    library writes through its raw address; a copy would leave the caller's
    tensor unfilled). Raises MambaScanError otherwise; returns t."""
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.device != device:
        raise _b.MambaScanError(7, "%s is on %s, expected %s" % (name, t.device, device))
    if t.dtype != dtype:
        raise _b.MambaScanError(3, "%s must be %s (got %s)" % (name, dtype, t.dtype))
    if tuple(t.shape) != tuple(shape):
        raise _b.MambaScanError(2, "%s must be %s (got %s)" % (name, list(shape), list(t.shape)))
    if not t.is_contiguous():
        raise _b.MambaScanError(2, "%s must be contiguous" % name)
    return t


def check_workspace(ws, device):
    """A caller-supplied workspace: a contiguous tensor on `device` (any dtype;
    its size in bytes is passed to the library, which checks it)."""
    if ws is None:
        return None
    if not isinstance(ws, torch.Tensor):
        raise TypeError("workspace must be a torch.Tensor")
    if ws.device != device:
        raise _b.MambaScanError(7, "workspace is on %s, expected %s" % (ws.device, device))
    if not ws.is_contiguous():
        raise _b.MambaScanError(6, "workspace must be contiguous")
    return ws


def _io(x):
    if x.dtype not in _IO:
        raise TypeError("io tensors must be float32 or bfloat16 (got %s)" % x.dtype)
    return _IO[x.dtype]


def workspace_bytes(batch, seqlen, d_inner, d_state, dtype, testing_kind=None):
    if testing_kind is not None:
        return _b.mamba_scan_testing_fwd_workspace_bytes(TESTING_KINDS[testing_kind], batch, seqlen, d_inner, d_state,
                                                         _IO[dtype])
    return _b.mamba_scan_fwd_workspace_bytes(batch, seqlen, d_inner, d_state, _IO[dtype])


def ckpt_like(x):
    """A float32 checkpoint tensor [batch, ceil(seqlen / 16), d_inner, 16] for `fwd(..., ckpt=)`
    and `bwd(..., ckpt=)` of inputs shaped like x [batch, seqlen, d_inner] (d_state 16)."""
    batch, seqlen, d_inner = x.shape
    return torch.empty(batch, (seqlen + 15) // 16, d_inner, 16, device=x.device, dtype=torch.float32)


# Kernel families of the testing entry point (include/mamba_scan_testing.h).
TESTING_KINDS = {"lane": 0, "quad": 1, "row": 2}


def fwd(x, dt, z, B, C, params, conv_state=None, ssm_state=None, *, out=None, conv_state_out=None,
        ssm_state_out=None, workspace=None, return_states=True, seq_idx=None, ckpt=None, testing_kind=None,
        testing_force_wide=False):
    """Prefill over x, dt, z [batch, seqlen, d_inner] and B, C [batch, seqlen, d_state].

    Returns (y, conv_state_out [batch, d_inner, 3], ssm_state_out [batch, d_inner, d_state]);
    the states are None when `return_states` is false. Preallocated outputs and
    workspace (a uint8 tensor) may be passed to avoid allocation. `seq_idx`
    ([batch, seqlen] integer document ids) packs documents: both states restart
    from zero wherever the id changes (mamba_scan_fwd_seq). `ckpt` (see
    `ckpt_like`; d_state 16, no seq_idx) is filled with the state before every
    16-step stage, which `bwd(..., ckpt=)` uses instead of recomputing it
    (mamba_scan_fwd_ckpt).

    Test suites only: `testing_kind` ("lane", "quad" or "row") and
    `testing_force_wide` route the call through mamba_scan_testing_fwd, which
    runs the chosen kernel family (and, for the sixteen-lane kernel, its
    per-stage-descriptor path) instead of the planned one.
    """
    io = _io(x)
    dtype = x.dtype
    x, dt, z = _dev(x, "x", dtype), _dev(dt, "dt", dtype), _dev(z, "z", dtype)
    B, C = _dev(B, "B", dtype), _dev(C, "C", dtype)
    f32 = torch.float32
    conv_w, conv_b = _dev(params.conv_w, "conv_w", f32), _dev(params.conv_b, "conv_b", f32)
    dt_bias, Dp, A = _dev(params.dt_bias, "dt_bias", f32), _dev(params.D, "D", f32), _dev(params.A, "A", f32)
    conv_state, ssm_state = _dev(conv_state, "conv_state", f32), _dev(ssm_state, "ssm_state", f32)
    if x.dim() != 3 or B.dim() != 3:
        raise _b.MambaScanError(2, "x must be [batch, seqlen, d_inner] and B [batch, seqlen, d_state]")
    batch, seqlen, d_inner = x.shape
    d_state = B.shape[2]
    d_conv = conv_w.shape[1] if conv_w.dim() == 2 else -1
    if dt.shape != x.shape or z.shape != x.shape or C.shape != B.shape or B.shape[:2] != x.shape[:2]:
        raise _b.MambaScanError(2, "shape mismatch between x/dt/z %s and B/C %s" % (tuple(x.shape), tuple(B.shape)))
    if (conv_w.shape[0] != d_inner or conv_b.shape != (d_inner,) or dt_bias.shape != (d_inner,)
            or Dp.shape != (d_inner,) or A.shape != (d_inner, d_state)):
        raise _b.MambaScanError(2, "parameter shapes do not match d_inner=%d d_state=%d" % (d_inner, d_state))
    if conv_state is not None and conv_state.shape != (batch, d_inner, d_conv - 1):
        raise _b.MambaScanError(2, "conv_state must be [%d, %d, %d]" % (batch, d_inner, d_conv - 1))
    if ssm_state is not None and ssm_state.shape != (batch, d_inner, d_state):
        raise _b.MambaScanError(2, "ssm_state must be [%d, %d, %d]" % (batch, d_inner, d_state))
    dev = x.device
    y = check_out(out, "out", x.shape, dtype, dev) if out is not None else torch.empty_like(x)
    if conv_state_out is not None:
        check_out(conv_state_out, "conv_state_out", (batch, d_inner, max(d_conv - 1, 0)), f32, dev)
    if ssm_state_out is not None:
        check_out(ssm_state_out, "ssm_state_out", (batch, d_inner, d_state), f32, dev)
    if return_states:
        if conv_state_out is None:
            conv_state_out = torch.empty(batch, d_inner, max(d_conv - 1, 0), device=dev, dtype=f32)
        if ssm_state_out is None:
            ssm_state_out = torch.empty(batch, d_inner, d_state, device=dev, dtype=f32)
    workspace = check_workspace(workspace, dev)
    testing = testing_kind is not None or testing_force_wide
    kind = -1 if testing_kind is None else TESTING_KINDS[testing_kind]
    if testing:
        ws_need = _b.mamba_scan_testing_fwd_workspace_bytes(kind, batch, seqlen, d_inner, d_state, io)
    else:
        ws_need = _b.mamba_scan_fwd_workspace_bytes(batch, seqlen, d_inner, d_state, io)
    if workspace is None and ws_need:
        workspace = torch.empty(ws_need, device=x.device, dtype=torch.uint8)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    stream = torch.cuda.current_stream(x.device).cuda_stream
    if seq_idx is not None:
        if isinstance(seq_idx, torch.Tensor) and seq_idx.dtype in (torch.int64, torch.int16, torch.int8, torch.uint8):
            seq_idx = seq_idx.to(torch.int32)
        seq_idx = _dev(seq_idx, "seq_idx", torch.int32)
        if seq_idx.shape != (batch, seqlen):
            raise _b.MambaScanError(2, "seq_idx must be [%d, %d]" % (batch, seqlen))
    if ckpt is not None:
        if seq_idx is not None:
            raise _b.MambaScanError(2, "checkpoints are not produced over packed documents")
        check_out(ckpt, "ckpt", (batch, (seqlen + 15) // 16, d_inner, 16), f32, dev)
    if testing:
        _b.mamba_scan_testing_fwd(kind, 1 if testing_force_wide else 0, batch, seqlen, d_inner, d_state, d_conv, io,
                                  _addr(x), _addr(dt), _addr(z), _addr(B), _addr(C), _addr(seq_idx), _addr(conv_w),
                                  _addr(conv_b), _addr(dt_bias), _addr(Dp), _addr(A), _addr(conv_state),
                                  _addr(ssm_state), _addr(y), _addr(conv_state_out), _addr(ssm_state_out),
                                  _addr(ckpt), _addr(workspace), ws_bytes, stream)
    elif ckpt is not None:
        _b.mamba_scan_fwd_ckpt(batch, seqlen, d_inner, d_state, d_conv, io, _addr(x), _addr(dt), _addr(z), _addr(B),
                               _addr(C), _addr(conv_w), _addr(conv_b), _addr(dt_bias), _addr(Dp), _addr(A),
                               _addr(conv_state), _addr(ssm_state), _addr(y), _addr(conv_state_out),
                               _addr(ssm_state_out), _addr(ckpt), _addr(workspace), ws_bytes, stream)
    elif seq_idx is None:
        _b.mamba_scan_fwd(batch, seqlen, d_inner, d_state, d_conv, io, _addr(x), _addr(dt), _addr(z), _addr(B),
                          _addr(C), _addr(conv_w), _addr(conv_b), _addr(dt_bias), _addr(Dp), _addr(A),
                          _addr(conv_state), _addr(ssm_state), _addr(y), _addr(conv_state_out),
                          _addr(ssm_state_out), _addr(workspace), ws_bytes, stream)
    else:
        _b.mamba_scan_fwd_seq(batch, seqlen, d_inner, d_state, d_conv, io, _addr(x), _addr(dt), _addr(z),
                              _addr(B), _addr(C), _addr(seq_idx), _addr(conv_w), _addr(conv_b), _addr(dt_bias),
                              _addr(Dp), _addr(A), _addr(conv_state), _addr(ssm_state), _addr(y),
                              _addr(conv_state_out), _addr(ssm_state_out), _addr(workspace), ws_bytes, stream)
    return y, conv_state_out, ssm_state_out


def bwd(x, dt, z, B, C, params, dy, conv_state=None, ssm_state=None, *, workspace=None, ckpt=None):
    """Gradients of `fwd` (without seq_idx) given dy = dL/dy [batch, seqlen, d_inner].

    Returns a dict: dx, ddt, dz (dtype and shape of x), dB, dC ([batch, seqlen,
    d_state] float32) and dconv_w, dconv_b, ddt_bias, dD, dA (float32, shapes of
    the parameters). The initial states enter the forward but get no gradient.
    d_state must be 16. With `ckpt` from `fwd(..., ckpt=)` of the same inputs
    the forward's states are not recomputed (mamba_scan_bwd_ckpt).
    """
    io = _io(x)
    dtype = x.dtype
    x, dt, z = _dev(x, "x", dtype), _dev(dt, "dt", dtype), _dev(z, "z", dtype)
    B, C, dy = _dev(B, "B", dtype), _dev(C, "C", dtype), _dev(dy, "dy", dtype)
    f32 = torch.float32
    conv_w, conv_b = _dev(params.conv_w, "conv_w", f32), _dev(params.conv_b, "conv_b", f32)
    dt_bias, Dp, A = _dev(params.dt_bias, "dt_bias", f32), _dev(params.D, "D", f32), _dev(params.A, "A", f32)
    conv_state, ssm_state = _dev(conv_state, "conv_state", f32), _dev(ssm_state, "ssm_state", f32)
    if x.dim() != 3 or B.dim() != 3:
        raise _b.MambaScanError(2, "x must be [batch, seqlen, d_inner] and B [batch, seqlen, d_state]")
    batch, seqlen, d_inner = x.shape
    d_state = B.shape[2]
    d_conv = conv_w.shape[1] if conv_w.dim() == 2 else -1
    if (dt.shape != x.shape or z.shape != x.shape or dy.shape != x.shape or C.shape != B.shape
            or B.shape[:2] != x.shape[:2]):
        raise _b.MambaScanError(2, "shape mismatch between x/dt/z/dy %s and B/C %s" % (tuple(x.shape),
                                                                                     tuple(B.shape)))
    if (conv_w.shape[0] != d_inner or conv_b.shape != (d_inner,) or dt_bias.shape != (d_inner,)
            or Dp.shape != (d_inner,) or A.shape != (d_inner, d_state)):
        raise _b.MambaScanError(2, "parameter shapes do not match d_inner=%d d_state=%d" % (d_inner, d_state))
    if conv_state is not None and conv_state.shape != (batch, d_inner, d_conv - 1):
        raise _b.MambaScanError(2, "conv_state must be [%d, %d, %d]" % (batch, d_inner, d_conv - 1))
    if ssm_state is not None and ssm_state.shape != (batch, d_inner, d_state):
        raise _b.MambaScanError(2, "ssm_state must be [%d, %d, %d]" % (batch, d_inner, d_state))
    dev = x.device
    g = dict(dx=torch.empty_like(x), ddt=torch.empty_like(x), dz=torch.empty_like(x),
             dB=torch.empty(B.shape, device=dev, dtype=f32), dC=torch.empty(B.shape, device=dev, dtype=f32),
             dconv_w=torch.empty(conv_w.shape, device=dev, dtype=f32), dconv_b=torch.empty_like(conv_b),
             ddt_bias=torch.empty_like(dt_bias), dD=torch.empty_like(Dp), dA=torch.empty_like(A))
    workspace = check_workspace(workspace, dev)
    if ckpt is not None:
        ckpt = _dev(ckpt, "ckpt", f32)
        if ckpt.shape != (batch, (seqlen + 15) // 16, d_inner, 16):
            raise _b.MambaScanError(2, "ckpt must be [%d, %d, %d, 16]" % (batch, (seqlen + 15) // 16, d_inner))
        ws_need = _b.mamba_scan_bwd_ckpt_workspace_bytes(batch, seqlen, d_inner, d_state, io)
    else:
        ws_need = _b.mamba_scan_bwd_workspace_bytes(batch, seqlen, d_inner, d_state, io)
    if workspace is None and ws_need:
        workspace = torch.empty(ws_need, device=dev, dtype=torch.uint8)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    stream = torch.cuda.current_stream(dev).cuda_stream
    grads = tuple(_addr(g[k]) for k in ("dx", "ddt", "dz", "dB", "dC", "dconv_w", "dconv_b", "ddt_bias", "dD", "dA"))
    common = (batch, seqlen, d_inner, d_state, d_conv, io, _addr(x), _addr(dt), _addr(z), _addr(B), _addr(C),
              _addr(conv_w), _addr(conv_b), _addr(dt_bias), _addr(Dp), _addr(A), _addr(conv_state),
              _addr(ssm_state), _addr(dy)) + grads
    if ckpt is not None:
        _b.mamba_scan_bwd_ckpt(*common, _addr(ckpt), _addr(workspace), ws_bytes, stream)
    else:
        _b.mamba_scan_bwd(*common, _addr(workspace), ws_bytes, stream)
    return g


def step(x, dt, z, B, C, params, conv_state, ssm_state, *, inplace=False, out=None):
    """One token: x, dt, z [batch, d_inner], B, C [batch, d_state]; states required.

    Functional by default (new state tensors are returned); with inplace=True the
    given state tensors are updated and returned.
    """
    io = _io(x)
    dtype = x.dtype
    x, dt, z = _dev(x, "x", dtype), _dev(dt, "dt", dtype), _dev(z, "z", dtype)
    B, C = _dev(B, "B", dtype), _dev(C, "C", dtype)
    f32 = torch.float32
    conv_w, conv_b = _dev(params.conv_w, "conv_w", f32), _dev(params.conv_b, "conv_b", f32)
    dt_bias, Dp, A = _dev(params.dt_bias, "dt_bias", f32), _dev(params.D, "D", f32), _dev(params.A, "A", f32)
    if conv_state is None or ssm_state is None:
        raise _b.MambaScanError(1, "step needs conv_state and ssm_state")
    if inplace and not (conv_state.is_contiguous() and ssm_state.is_contiguous()):
        raise _b.MambaScanError(2, "in-place step needs contiguous state tensors")
    conv_state, ssm_state = _dev(conv_state, "conv_state", f32), _dev(ssm_state, "ssm_state", f32)
    if x.dim() != 2 or B.dim() != 2:
        raise _b.MambaScanError(2, "x must be [batch, d_inner] and B [batch, d_state]")
    batch, d_inner = x.shape
    d_state = B.shape[1]
    d_conv = conv_w.shape[1] if conv_w.dim() == 2 else -1
    if dt.shape != x.shape or z.shape != x.shape or C.shape != B.shape or B.shape[0] != batch:
        raise _b.MambaScanError(2, "shape mismatch between x/dt/z and B/C")
    if (conv_w.shape[0] != d_inner or conv_b.shape != (d_inner,) or dt_bias.shape != (d_inner,)
            or Dp.shape != (d_inner,) or A.shape != (d_inner, d_state)):
        raise _b.MambaScanError(2, "parameter shapes do not match d_inner=%d d_state=%d" % (d_inner, d_state))
    if conv_state.shape != (batch, d_inner, d_conv - 1) or ssm_state.shape != (batch, d_inner, d_state):
        raise _b.MambaScanError(2, "state shapes do not match")
    y = check_out(out, "out", x.shape, dtype, x.device) if out is not None else torch.empty_like(x)
    if inplace:
        cso, sso = conv_state, ssm_state
    else:
        cso, sso = torch.empty_like(conv_state), torch.empty_like(ssm_state)
    stream = torch.cuda.current_stream(x.device).cuda_stream
    _b.mamba_scan_step(batch, d_inner, d_state, d_conv, io, _addr(x), _addr(dt), _addr(z), _addr(B), _addr(C),
                       _addr(conv_w), _addr(conv_b), _addr(dt_bias), _addr(Dp), _addr(A), _addr(conv_state),
                       _addr(ssm_state), _addr(y), _addr(cso), _addr(sso), stream)
    return y, cso, sso
