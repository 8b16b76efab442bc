"""fp64 CPU oracle of the Mamba-1 selective-scan mixer core.

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg use it; the HIP product path never imports it and shares no
code with it.

`oracle_fwd` runs the whole sequence and `oracle_step` one token, each
following calm-mamba 0.1.4 PKG-INFO ("Mamba operator", steps 2 and 4-6):
causal depthwise conv + SiLU, softplus step size, the recurrence
h = exp(delta*A)*h + delta*B*x with readout C.h + D*x, and the SiLU(z) gate.
Inputs are upcast to float64 (exact for fp32 and bf16 values), so the oracle
sees exactly the numbers the GPU sees.
"""
import ctypes
import os

import numpy as np

from . import build as _build

_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        _lib = load_library(_build.LIB)
    return _lib


def load_library(path):
    """Load an oracle shared library at `path` and declare its signatures."""
    lib = ctypes.CDLL(path)
    i64 = ctypes.c_int64
    dp = ctypes.POINTER(ctypes.c_double)
    lib.oracle_fwd.restype = ctypes.c_int
    lib.oracle_fwd.argtypes = [i64] * 5 + [dp] * 15 + [ctypes.c_int]
    lib.oracle_fwd_seq.restype = ctypes.c_int
    lib.oracle_fwd_seq.argtypes = [i64] * 5 + [dp] * 10 + [ctypes.POINTER(ctypes.c_int32)] + [dp] * 5 + [ctypes.c_int]
    lib.oracle_bwd.restype = ctypes.c_int
    lib.oracle_bwd.argtypes = [i64] * 5 + [dp] * 23 + [ctypes.c_int]
    lib.oracle_fwd_xc.restype = ctypes.c_int
    lib.oracle_fwd_xc.argtypes = [i64] * 4 + [dp] * 11
    lib.oracle_step.restype = ctypes.c_int
    lib.oracle_step.argtypes = [i64] * 4 + [dp] * 15
    return lib


def _f64(a):
    """Contiguous float64 numpy copy of a numpy array or torch tensor."""
    if a is None:
        return None
    if hasattr(a, "detach"):  # torch tensor: upcast through float32 (exact for bf16/fp32)
        a = a.detach().cpu()
        a = a.double().numpy()
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _ptr(a):
    if a is None:
        return ctypes.POINTER(ctypes.c_double)()
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def oracle_fwd(x, dt, z, B, C, conv_w, conv_b, dt_bias, D, A, conv_state=None, ssm_state=None,
               nthreads=0, lib=None, seq_idx=None):
    """Prefill over a whole sequence.

    x, dt, z: [batch, seqlen, d_inner]; B, C: [batch, seqlen, d_state];
    conv_w: [d_inner, d_conv]; conv_b, dt_bias, D: [d_inner]; A: [d_inner, d_state];
    conv_state: [batch, d_inner, d_conv-1] or None; ssm_state: [batch, d_inner, d_state] or None;
    seq_idx: [batch, seqlen] integer document ids or None (both states reset to
    zero wherever the id changes along t).
    Returns float64 arrays (y, conv_state_out, ssm_state_out).
    """
    lib = lib or _load()
    x, dt, z, B, C = map(_f64, (x, dt, z, B, C))
    conv_w, conv_b, dt_bias, D, A = map(_f64, (conv_w, conv_b, dt_bias, D, A))
    cs, ss = _f64(conv_state), _f64(ssm_state)
    batch, seqlen, d_inner = x.shape
    d_state = B.shape[2]
    d_conv = conv_w.shape[1]
    assert dt.shape == x.shape and z.shape == x.shape
    assert B.shape == (batch, seqlen, d_state) and C.shape == B.shape
    assert conv_w.shape == (d_inner, d_conv) and A.shape == (d_inner, d_state)
    assert conv_b.shape == (d_inner,) and dt_bias.shape == (d_inner,) and D.shape == (d_inner,)
    if cs is not None:
        assert cs.shape == (batch, d_inner, d_conv - 1)
    if ss is not None:
        assert ss.shape == (batch, d_inner, d_state)
    y = np.empty_like(x)
    cso = np.empty((batch, d_inner, d_conv - 1))
    sso = np.empty((batch, d_inner, d_state))
    if seq_idx is None:
        rc = lib.oracle_fwd(batch, seqlen, d_inner, d_state, d_conv, _ptr(x), _ptr(dt), _ptr(z), _ptr(B),
                            _ptr(C), _ptr(conv_w), _ptr(conv_b), _ptr(dt_bias), _ptr(D), _ptr(A), _ptr(cs),
                            _ptr(ss), _ptr(y), _ptr(cso), _ptr(sso), int(nthreads))
    else:
        if hasattr(seq_idx, "detach"):
            seq_idx = seq_idx.detach().cpu().numpy()
        sq = np.ascontiguousarray(np.asarray(seq_idx), dtype=np.int32)
        assert sq.shape == (batch, seqlen)
        rc = lib.oracle_fwd_seq(batch, seqlen, d_inner, d_state, d_conv, _ptr(x), _ptr(dt), _ptr(z), _ptr(B),
                                _ptr(C), _ptr(conv_w), _ptr(conv_b), _ptr(dt_bias), _ptr(D), _ptr(A),
                                sq.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), _ptr(cs), _ptr(ss), _ptr(y),
                                _ptr(cso), _ptr(sso), int(nthreads))
    if rc != 0:
        raise ValueError("oracle_fwd rejected its arguments")
    return y, cso, sso


def oracle_fwd_xc(xc, dt, z, B, C, dt_bias, D, A, ssm_state=None, lib=None):
    """Prefill from a given activated conv output xc [batch, seqlen, d_inner]
    (no conv inside; see oracle_fwd_xc in mamba_oracle.c). Returns float64
    (y, ssm_state_out)."""
    lib = lib or _load()
    xc, dt, z, B, C = map(_f64, (xc, dt, z, B, C))
    dt_bias, D, A, ss = map(_f64, (dt_bias, D, A, ssm_state))
    batch, seqlen, d_inner = xc.shape
    d_state = B.shape[2]
    assert dt.shape == xc.shape and z.shape == xc.shape and B.shape == (batch, seqlen, d_state) and C.shape == B.shape
    assert dt_bias.shape == (d_inner,) and D.shape == (d_inner,) and A.shape == (d_inner, d_state)
    if ss is not None:
        assert ss.shape == (batch, d_inner, d_state)
    y = np.empty_like(xc)
    sso = np.empty((batch, d_inner, d_state))
    rc = lib.oracle_fwd_xc(batch, seqlen, d_inner, d_state, _ptr(xc), _ptr(dt), _ptr(z), _ptr(B), _ptr(C),
                           _ptr(dt_bias), _ptr(D), _ptr(A), _ptr(ss), _ptr(y), _ptr(sso))
    if rc != 0:
        raise ValueError("oracle_fwd_xc rejected its arguments")
    return y, sso


def oracle_step(x, dt, z, B, C, conv_w, conv_b, dt_bias, D, A, conv_state, ssm_state, lib=None):
    """One token per batch row. x, dt, z: [batch, d_inner]; B, C: [batch, d_state];
    states as in `oracle_fwd` (required). Returns float64 (y, conv_state', ssm_state')."""
    lib = lib or _load()
    x, dt, z, B, C = map(_f64, (x, dt, z, B, C))
    conv_w, conv_b, dt_bias, D, A = map(_f64, (conv_w, conv_b, dt_bias, D, A))
    cs, ss = _f64(conv_state), _f64(ssm_state)
    batch, d_inner = x.shape
    d_state = B.shape[1]
    d_conv = conv_w.shape[1]
    assert cs.shape == (batch, d_inner, d_conv - 1) and ss.shape == (batch, d_inner, d_state)
    y = np.empty_like(x)
    cso = np.empty_like(cs)
    sso = np.empty_like(ss)
    rc = lib.oracle_step(batch, d_inner, d_state, d_conv, _ptr(x), _ptr(dt), _ptr(z), _ptr(B), _ptr(C),
                         _ptr(conv_w), _ptr(conv_b), _ptr(dt_bias), _ptr(D), _ptr(A), _ptr(cs), _ptr(ss),
                         _ptr(y), _ptr(cso), _ptr(sso))
    if rc != 0:
        raise ValueError("oracle_step rejected its arguments")
    return y, cso, sso


def oracle_bwd(x, dt, z, B, C, conv_w, conv_b, dt_bias, D, A, dy, conv_state=None, ssm_state=None, nthreads=0,
               lib=None):
    """Gradients of the prefill given dy = dL/dy [batch, seqlen, d_inner]. Returns a dict of
    float64 arrays: dx, ddt, dz (like x), dB, dC (like B), dconv_w, dconv_b, ddt_bias, dD, dA
    (like the parameters). The initial states enter the forward but get no gradient."""
    lib = lib or _load()
    x, dt, z, B, C, dy = map(_f64, (x, dt, z, B, C, dy))
    conv_w, conv_b, dt_bias, D, A = map(_f64, (conv_w, conv_b, dt_bias, D, A))
    cs, ss = _f64(conv_state), _f64(ssm_state)
    batch, seqlen, d_inner = x.shape
    d_state = B.shape[2]
    d_conv = conv_w.shape[1]
    assert dy.shape == x.shape
    g = dict(dx=np.empty_like(x), ddt=np.empty_like(x), dz=np.empty_like(x), dB=np.empty_like(B),
             dC=np.empty_like(B), dconv_w=np.empty_like(conv_w), dconv_b=np.empty_like(conv_b),
             ddt_bias=np.empty_like(dt_bias), dD=np.empty_like(D), dA=np.empty_like(A))
    rc = lib.oracle_bwd(batch, seqlen, d_inner, d_state, d_conv, _ptr(x), _ptr(dt), _ptr(z), _ptr(B), _ptr(C),
                        _ptr(conv_w), _ptr(conv_b), _ptr(dt_bias), _ptr(D), _ptr(A), _ptr(cs), _ptr(ss), _ptr(dy),
                        *(_ptr(g[k]) for k in ("dx", "ddt", "dz", "dB", "dC", "dconv_w", "dconv_b", "ddt_bias",
                                               "dD", "dA")), int(nthreads))
    if rc != 0:
        raise ValueError("oracle_bwd rejected its arguments")
    return g
