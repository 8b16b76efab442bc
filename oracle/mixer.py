"""fp64 oracle of one Mamba-1 mixer layer (TEST INFRASTRUCTURE ONLY, like the
rest of this package: only the tests, the smoke check and the benchmark's
CPU-baseline leg use it).

calm-mamba 0.1.4 PKG-INFO, "Architecture" / "Mamba operator", steps 1-7, in
order: in_proj splits the input into the SSM branch x and the gate branch z;
causal depthwise conv (kernel 4) + SiLU gives xc; x_proj maps xc to the
input-dependent dt (through a dt_rank bottleneck), B and C; dt_proj and
softplus give the step sizes; the selective scan and readout; the SiLU(z)
gate; the bias-free output projection. The projections are numpy matmuls in
float64; the conv + SiLU of step 2 is written out here (x_proj consumes xc)
and steps 4-6 of the whole sequence are the pinned scan oracle fed that xc
(`oracle_fwd_xc`), as step 5 uses step 2's output; the conv state is the
last three entries of (history ++ x). The one-token step is the same with
the window (conv state ++ x) and a sequence of length one. Nothing is
rounded between steps.

With `io_dtype=torch.bfloat16` the oracle rounds each intermediate (x, z,
xc, dt_low, B, C, dt, y) to bfloat16 (round to nearest even) at the point
where the GPU layer stores it in that dtype, and the later steps use the
rounded value (the reading the layer's header states: intermediates are
kept in the io dtype); the arithmetic between those points stays float64.
Without it nothing is rounded: the exact layer, against which the tests
also report (and bound) the bfloat16 layer's error.

Weights use the torch Linear layout [out_features, in_features]: w_in
[2*d_inner, d_model] (x rows first), w_x [dt_rank + 2*d_state, d_inner] (dt
rows, then B, then C), w_dt [d_inner, dt_rank], w_out [d_model, d_inner].
"""
import numpy as np
import torch

from . import _f64, oracle_fwd_xc


def _rounder(io_dtype):
    if io_dtype is None or io_dtype == torch.float64:
        return lambda a: a
    return lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(io_dtype).double().numpy()


def _silu(u):
    return u / (1.0 + np.exp(-u))


def _split(w_x, dt_rank, d_state):
    return w_x[:dt_rank], w_x[dt_rank:dt_rank + d_state], w_x[dt_rank + d_state:dt_rank + 2 * d_state]


def mixer_fwd(hidden, w_in, conv_w, conv_b, w_x, w_dt, dt_bias, A, D, w_out, conv_state=None, ssm_state=None,
              lib=None, io_dtype=None):
    """hidden [batch, seqlen, d_model] -> float64 (out, conv_state', ssm_state')."""
    rd = _rounder(io_dtype)
    u, w_in, conv_w, conv_b, w_x, w_dt, w_out = map(_f64, (hidden, w_in, conv_w, conv_b, w_x, w_dt, w_out))
    d_inner = w_in.shape[0] // 2
    dt_rank = w_dt.shape[1]
    d_state = (w_x.shape[0] - dt_rank) // 2
    batch, seqlen, _ = u.shape
    # 1 in_proj
    x = rd(u @ w_in[:d_inner].T)
    z = rd(u @ w_in[d_inner:].T)
    # 2 conv over (history ++ x), tap 3 on the newest token, then SiLU
    hist = np.zeros((batch, 3, d_inner)) if conv_state is None else np.transpose(_f64(conv_state), (0, 2, 1))
    xw = np.concatenate([hist, x], axis=1)
    pre = conv_b[None, None, :] + sum(conv_w[None, None, :, k] * xw[:, k:k + seqlen, :] for k in range(4))
    xc = rd(_silu(pre))
    # 3 x_proj
    w_dtl, w_B, w_C = _split(w_x, dt_rank, d_state)
    dt_low, B, C = rd(xc @ w_dtl.T), rd(xc @ w_B.T), rd(xc @ w_C.T)
    # 4 dt_proj (softplus and dt_bias inside the scan oracle)
    dt = rd(dt_low @ w_dt.T)
    # 4-6 scan with gate, from xc
    y, ss = oracle_fwd_xc(xc, dt, z, B, C, dt_bias, D, A, ssm_state, lib=lib)
    # conv state: the last three entries of (history ++ x), oldest first
    cs = np.transpose(xw[:, -3:, :], (0, 2, 1)).copy()
    # 7 out_proj
    return rd(y) @ w_out.T, cs, ss


def mixer_step(hidden, w_in, conv_w, conv_b, w_x, w_dt, dt_bias, A, D, w_out, conv_state, ssm_state, lib=None,
               io_dtype=None):
    """One token per batch row: hidden [batch, d_model] -> float64 (out, conv_state', ssm_state')."""
    rd = _rounder(io_dtype)
    u, w_in, conv_w, conv_b, w_x, w_dt, w_out = map(_f64, (hidden, w_in, conv_w, conv_b, w_x, w_dt, w_out))
    cs = _f64(conv_state)
    d_inner = w_in.shape[0] // 2
    dt_rank = w_dt.shape[1]
    d_state = (w_x.shape[0] - dt_rank) // 2
    x = rd(u @ w_in[:d_inner].T)
    z = rd(u @ w_in[d_inner:].T)
    # the window is (conv_state[0], conv_state[1], conv_state[2], x)
    pre = conv_b + conv_w[:, 3] * x + sum(conv_w[:, k] * cs[:, :, k] for k in range(3))
    xc = rd(_silu(pre))
    w_dtl, w_B, w_C = _split(w_x, dt_rank, d_state)
    dt = rd(rd(xc @ w_dtl.T) @ w_dt.T)
    # 4-6 for the one token from xc: the scan oracle over a sequence of length one
    y, ss2 = oracle_fwd_xc(xc[:, None], dt[:, None], z[:, None], rd(xc @ w_B.T)[:, None], rd(xc @ w_C.T)[:, None],
                           dt_bias, D, A, ssm_state, lib=lib)
    # the new conv state drops the oldest entry and appends x
    cs2 = np.concatenate([cs[:, :, 1:], x[:, :, None]], axis=2)
    return rd(y[:, 0]) @ w_out.T, cs2, ss2
