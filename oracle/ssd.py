"""fp64 CPU oracle of the Mamba-2 SSD scan (scalar decay per head).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg use it; the HIP product path never imports it and shares no
code with it.

`oracle_ssd_fwd` runs the whole sequence and `oracle_ssd_step` one token
(niverel-mamba 0.1.0 PKG-INFO, "The weight contract" and "Autoregressive
decoding"): delta = softplus(dt + dt_bias), S = exp(delta A) S + delta x B^T,
y = S C + D x per head, with B and C shared by a group of heads. Inputs are
upcast to float64 (exact for fp32 and bf16 values).
"""
import ctypes
import os

import numpy as np

from . import build as _build

_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_build.SSD_LIB):
            _build.build(_build.SSD_SRC, _build.SSD_LIB)
        _lib = load_library(_build.SSD_LIB)
    return _lib


def load_library(path):
    """Load an SSD oracle shared library at `path` and declare its signatures."""
    lib = ctypes.CDLL(path)
    i64 = ctypes.c_int64
    dp = ctypes.POINTER(ctypes.c_double)
    lib.oracle_ssd_fwd.restype = ctypes.c_int
    lib.oracle_ssd_fwd.argtypes = [i64] * 6 + [dp] * 10 + [ctypes.c_int]
    lib.oracle_ssd_fwd_seq.restype = ctypes.c_int
    lib.oracle_ssd_fwd_seq.argtypes = [i64] * 6 + [dp] * 4 + [ctypes.POINTER(ctypes.c_int32)] + [dp] * 6 + [ctypes.c_int]
    lib.oracle_ssd_step.restype = ctypes.c_int
    lib.oracle_ssd_step.argtypes = [i64] * 5 + [dp] * 10
    return lib


def _f64(a):
    if a is None:
        return None
    if hasattr(a, "detach"):
        a = a.detach().cpu().double().numpy()
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _ptr(a):
    if a is None:
        return ctypes.POINTER(ctypes.c_double)()
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def oracle_ssd_fwd(x, dt, B, C, dt_bias, A, D, state=None, nthreads=0, lib=None, seq_idx=None):
    """x [batch, seqlen, nheads, headdim]; dt [batch, seqlen, nheads];
    B, C [batch, seqlen, ngroups, d_state]; dt_bias, A, D [nheads];
    state [batch, nheads, headdim, d_state] or None; seq_idx [batch, seqlen]
    integer document ids or None (the state restarts from zero wherever the id
    changes). Returns float64 arrays (y like x, final state)."""
    lib = lib or _load()
    x, dt, B, C, dt_bias, A, D, st = map(_f64, (x, dt, B, C, dt_bias, A, D, state))
    batch, seqlen, nheads, headdim = x.shape
    ngroups, d_state = B.shape[2], B.shape[3]
    assert dt.shape == (batch, seqlen, nheads) and B.shape == C.shape == (batch, seqlen, ngroups, d_state)
    y = np.empty_like(x)
    so = np.empty((batch, nheads, headdim, d_state))
    if seq_idx is None:
        rc = lib.oracle_ssd_fwd(batch, seqlen, nheads, headdim, d_state, ngroups, _ptr(x), _ptr(dt), _ptr(B),
                                _ptr(C), _ptr(dt_bias), _ptr(A), _ptr(D), _ptr(st), _ptr(y), _ptr(so), int(nthreads))
    else:
        if hasattr(seq_idx, "detach"):
            seq_idx = seq_idx.detach().cpu().numpy()
        ids = np.ascontiguousarray(np.asarray(seq_idx, dtype=np.int32))
        assert ids.shape == (batch, seqlen)
        rc = lib.oracle_ssd_fwd_seq(batch, seqlen, nheads, headdim, d_state, ngroups, _ptr(x), _ptr(dt), _ptr(B),
                                    _ptr(C), ids.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), _ptr(dt_bias),
                                    _ptr(A), _ptr(D), _ptr(st), _ptr(y), _ptr(so), int(nthreads))
    if rc != 0:
        raise ValueError("oracle_ssd_fwd rejected its arguments")
    return y, so


def oracle_ssd_step(x, dt, B, C, dt_bias, A, D, state, lib=None):
    """One token: x [batch, nheads, headdim], dt [batch, nheads], B, C [batch, ngroups, d_state],
    state [batch, nheads, headdim, d_state] (required). Returns (y, new state)."""
    lib = lib or _load()
    x, dt, B, C, dt_bias, A, D, st = map(_f64, (x, dt, B, C, dt_bias, A, D, state))
    batch, nheads, headdim = x.shape
    ngroups, d_state = B.shape[1], B.shape[2]
    y = np.empty_like(x)
    so = np.empty_like(st)
    rc = lib.oracle_ssd_step(batch, nheads, headdim, d_state, ngroups, _ptr(x), _ptr(dt), _ptr(B), _ptr(C),
                             _ptr(dt_bias), _ptr(A), _ptr(D), _ptr(st), _ptr(y), _ptr(so))
    if rc != 0:
        raise ValueError("oracle_ssd_step rejected its arguments")
    return y, so
