"""torch-tensor front end of the Mamba-2 SSD scan in libmamba_scan (`ssd_fwd`,
and `ssd_step` for one token).

Marshalling only: checks devices, dtypes and shapes, makes tensors contiguous,
allocates outputs and the workspace, and passes raw device addresses plus
torch's current HIP stream to mamba2_ssd_fwd. The arithmetic is all in the
library's kernels.
"""
import torch

from . import _binding as _b
from .api import _IO, _addr, _dev, _io, check_out, check_workspace


def ssd_workspace_bytes(batch, seqlen, nheads, headdim, d_state, ngroups, dtype):
    return _b.mamba2_ssd_fwd_workspace_bytes(batch, seqlen, nheads, headdim, d_state, ngroups, _IO[dtype])


def ssd_fwd(x, dt, B, C, dt_bias, A, D, state=None, *, out=None, state_out=None, workspace=None,
            return_state=True, seq_idx=None):
    """x [batch, seqlen, nheads, headdim]; dt [batch, seqlen, nheads] (before dt_bias and
    softplus); B, C [batch, seqlen, ngroups, d_state]; dt_bias, A, D [nheads] float32;
    state [batch, nheads, headdim, d_state] float32 or None; seq_idx [batch, seqlen]
    integer document ids or None (packed documents: the state restarts from zero
    wherever the id changes, mamba2_ssd_fwd_seq).
    Returns (y like x, final state or None)."""
    io = _io(x)
    dtype = x.dtype
    x, dt = _dev(x, "x", dtype), _dev(dt, "dt", dtype)
    B, C = _dev(B, "B", dtype), _dev(C, "C", dtype)
    f32 = torch.float32
    dt_bias, A, D = _dev(dt_bias, "dt_bias", f32), _dev(A, "A", f32), _dev(D, "D", f32)
    state = _dev(state, "state", f32)
    if x.dim() != 4 or B.dim() != 4:
        raise _b.MambaScanError(2, "x must be [batch, seqlen, nheads, headdim] and B [batch, seqlen, ngroups, d_state]")
    batch, seqlen, nheads, headdim = x.shape
    ngroups, d_state = B.shape[2], B.shape[3]
    if dt.shape != (batch, seqlen, nheads) or C.shape != B.shape or B.shape[:2] != (batch, seqlen):
        raise _b.MambaScanError(2, "shape mismatch between x %s, dt %s and B/C %s" % (tuple(x.shape), tuple(dt.shape),
                                                                                    tuple(B.shape)))
    if dt_bias.shape != (nheads,) or A.shape != (nheads,) or D.shape != (nheads,):
        raise _b.MambaScanError(2, "dt_bias, A and D must be [%d]" % nheads)
    if state is not None and state.shape != (batch, nheads, headdim, d_state):
        raise _b.MambaScanError(2, "state must be [%d, %d, %d, %d]" % (batch, nheads, headdim, d_state))
    y = check_out(out, "out", x.shape, dtype, x.device) if out is not None else torch.empty_like(x)
    if state_out is not None:
        check_out(state_out, "state_out", (batch, nheads, headdim, d_state), f32, x.device)
    if return_state and state_out is None:
        state_out = torch.empty(batch, nheads, headdim, d_state, device=x.device, dtype=f32)
    workspace = check_workspace(workspace, x.device)
    ws_need = _b.mamba2_ssd_fwd_workspace_bytes(batch, seqlen, nheads, headdim, d_state, ngroups, io)
    if workspace is None and ws_need:
        workspace = torch.empty(ws_need, device=x.device, dtype=torch.uint8)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    stream = torch.cuda.current_stream(x.device).cuda_stream
    if seq_idx is None:
        _b.mamba2_ssd_fwd(batch, seqlen, nheads, headdim, d_state, ngroups, io, _addr(x), _addr(dt), _addr(B),
                          _addr(C), _addr(dt_bias), _addr(A), _addr(D), _addr(state), _addr(y), _addr(state_out),
                          _addr(workspace), ws_bytes, stream)
    else:
        if isinstance(seq_idx, torch.Tensor) and seq_idx.dtype in (torch.int64, torch.int16, torch.int8, torch.uint8):
            seq_idx = seq_idx.to(torch.int32)
        seq_idx = _dev(seq_idx, "seq_idx", torch.int32)
        if seq_idx.shape != (batch, seqlen):
            raise _b.MambaScanError(2, "seq_idx must be [%d, %d]" % (batch, seqlen))
        _b.mamba2_ssd_fwd_seq(batch, seqlen, nheads, headdim, d_state, ngroups, io, _addr(x), _addr(dt), _addr(B),
                              _addr(C), _addr(seq_idx), _addr(dt_bias), _addr(A), _addr(D), _addr(state), _addr(y),
                              _addr(state_out), _addr(workspace), ws_bytes, stream)
    return y, state_out


def ssd_step(x, dt, B, C, dt_bias, A, D, state, *, inplace=False, out=None):
    """One token: x [batch, nheads, headdim], dt [batch, nheads], B, C [batch, ngroups,
    d_state], state [batch, nheads, headdim, d_state] float32 (required).
    Functional by default (a new state is returned); with inplace=True the given
    state is updated and returned."""
    io = _io(x)
    dtype = x.dtype
    x, dt = _dev(x, "x", dtype), _dev(dt, "dt", dtype)
    B, C = _dev(B, "B", dtype), _dev(C, "C", dtype)
    f32 = torch.float32
    dt_bias, A, D = _dev(dt_bias, "dt_bias", f32), _dev(A, "A", f32), _dev(D, "D", f32)
    if state is None:
        raise _b.MambaScanError(1, "ssd_step needs a state")
    if inplace and not state.is_contiguous():
        raise _b.MambaScanError(2, "in-place step needs a contiguous state tensor")
    state = _dev(state, "state", f32)
    if x.dim() != 3 or B.dim() != 3:
        raise _b.MambaScanError(2, "x must be [batch, nheads, headdim] and B [batch, ngroups, d_state]")
    batch, nheads, headdim = x.shape
    ngroups, d_state = B.shape[1], B.shape[2]
    if dt.shape != (batch, nheads) or C.shape != B.shape or B.shape[0] != batch:
        raise _b.MambaScanError(2, "shape mismatch between x, dt and B/C")
    if dt_bias.shape != (nheads,) or A.shape != (nheads,) or D.shape != (nheads,):
        raise _b.MambaScanError(2, "dt_bias, A and D must be [%d]" % nheads)
    if state.shape != (batch, nheads, headdim, d_state):
        raise _b.MambaScanError(2, "state must be [%d, %d, %d, %d]" % (batch, nheads, headdim, d_state))
    y = check_out(out, "out", x.shape, dtype, x.device) if out is not None else torch.empty_like(x)
    so = state if inplace else torch.empty_like(state)
    stream = torch.cuda.current_stream(x.device).cuda_stream
    _b.mamba2_ssd_step(batch, nheads, headdim, d_state, ngroups, io, _addr(x), _addr(dt), _addr(B), _addr(C),
                       _addr(dt_bias), _addr(A), _addr(D), _addr(state), _addr(y), _addr(so), stream)
    return y, so
