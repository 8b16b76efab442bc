"""Pins of the Mamba-2 SSD oracle: each compares `oracle.ssd` (loaded from a
given library, so that planted mutants can be checked too) with something
other than itself. Every pin returns the worst scaled error it saw; the bound
is PIN_TOL unless a pin says otherwise.

- dual:     the quadratic (attention-like) form, non-recursive, in numpy:
            y_t = sum_{s<=t} (C_t . B_s) exp(A sum_{s<r<=t} delta_r) delta_s x_s
                  + C_t . exp(A sum_{r<=t} delta_r) S0 + D x_t,
            with delta = numpy.logaddexp(0, dt + dt_bias), two groups of heads;
- a_zero:   A = 0 gives S_t = S0 + cumsum_s(delta_s x_s B_s^T) (numpy.cumsum);
- no_step:  delta = 0 (dt_bias = -1e4) gives y = C.S0 + D x and S unchanged;
- iir:      one head, headdim 1, d_state 1, B = C = 1, constant delta: the
            state is scipy.signal.lfilter([delta], [1, -e^{delta A}], x);
- steps:    oracle_ssd_step applied token by token equals oracle_ssd_fwd;
- resume:   fwd(x[:k]) then fwd(x[k:], state) equals fwd(x);
- packed:   packed documents (seq_idx) equal each document run on its own.
"""
import numpy as np
import scipy.signal
import torch

import workloads
from oracle import ssd

PIN_TOL = 1e-12


def scaled_err(got, want):
    got, want = np.atleast_1d(np.asarray(got, np.float64)), np.atleast_1d(np.asarray(want, np.float64))
    rms = float(np.sqrt(np.mean(want * want))) if want.size else 0.0
    scale = np.maximum(np.abs(want), rms)
    scale[scale == 0] = 1.0
    return float((np.abs(got - want) / scale).max()) if want.size else 0.0


def _np(lay):
    return {k: v.double().numpy() for k, v in lay.items()}


def _delta(dt, dt_bias):
    return np.logaddexp(0.0, dt + dt_bias[None, None, :])


def dual_form(lay, S0=None):
    """numpy quadratic form; returns (y, final state)."""
    a = _np(lay)
    x, dt, B, C, A, D = a["x"], a["dt"], a["B"], a["C"], a["A"], a["D"]
    b_, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    hpg = H // G
    delta = _delta(dt, a["dt_bias"])
    y = np.zeros_like(x)
    Sf = np.zeros((b_, H, P, N))
    for b in range(b_):
        for h in range(H):
            g = h // hpg
            dl = delta[b, :, h]
            for t in range(L):
                acc = D[h] * x[b, t, h]
                for s in range(t + 1):
                    w = np.exp(A[h] * dl[s + 1:t + 1].sum()) * dl[s] * (C[b, t, g] @ B[b, s, g])
                    acc = acc + w * x[b, s, h]
                if S0 is not None:
                    acc = acc + np.exp(A[h] * dl[:t + 1].sum()) * (S0[b, h] @ C[b, t, g])
                y[b, t, h] = acc
            S = np.zeros((P, N)) if S0 is None else np.exp(A[h] * dl.sum()) * S0[b, h]
            for s in range(L):
                S = S + np.exp(A[h] * dl[s + 1:].sum()) * dl[s] * np.outer(x[b, s, h], B[b, s, g])
            Sf[b, h] = S
    return y, Sf


def pin_dual(lib):
    worst = 0.0
    for seed, (b, L, H, P, N, G), with_state in [(1, (2, 9, 4, 3, 5, 2), True), (2, (1, 12, 2, 4, 3, 1), False)]:
        lay = workloads.make_ssd(b, L, H, P, N, G, torch.float32, seed=seed, dt_range=(1e-2, 5e-1))
        S0 = np.random.default_rng(seed).standard_normal((b, H, P, N)) if with_state else None
        y, s = ssd.oracle_ssd_fwd(*(lay[k] for k in workloads.SSD_KEYS), state=S0, lib=lib)
        yd, sd = dual_form(lay, S0)
        worst = max(worst, scaled_err(y, yd), scaled_err(s, sd))
    return worst


def pin_a_zero(lib):
    lay = workloads.make_ssd(2, 11, 3, 4, 6, 1, torch.float32, seed=3)
    lay["A"] = torch.zeros_like(lay["A"])
    S0 = np.random.default_rng(3).standard_normal((2, 3, 4, 6))
    y, s = ssd.oracle_ssd_fwd(*(lay[k] for k in workloads.SSD_KEYS), state=S0, lib=lib)
    a = _np(lay)
    delta = _delta(a["dt"], a["dt_bias"])
    inc = delta[..., None, None] * a["x"][..., :, None] * a["B"][:, :, 0, None, None, :]  # [b, t, h, p, n]
    S = S0[:, None] + np.cumsum(inc, axis=1)
    yw = np.einsum("bthpn,btn->bthp", S, a["C"][:, :, 0]) + a["D"][None, None, :, None] * a["x"]
    return max(scaled_err(y, yw), scaled_err(s, S[:, -1]))


def pin_no_step(lib):
    lay = workloads.make_ssd(2, 7, 2, 3, 4, 1, torch.float32, seed=4)
    lay["dt_bias"] = torch.full_like(lay["dt_bias"], -1e4)
    S0 = np.random.default_rng(4).standard_normal((2, 2, 3, 4))
    y, s = ssd.oracle_ssd_fwd(*(lay[k] for k in workloads.SSD_KEYS), state=S0, lib=lib)
    a = _np(lay)
    yw = np.einsum("bhpn,btn->bthp", S0, a["C"][:, :, 0]) + a["D"][None, None, :, None] * a["x"]
    return max(scaled_err(y, yw), scaled_err(s, S0))


def pin_iir(lib):
    L = 50
    lay = workloads.make_ssd(1, L, 1, 1, 1, 1, torch.float32, seed=5, dt_range=(0.05, 0.3))
    lay["dt"] = torch.zeros_like(lay["dt"])
    lay["B"] = torch.ones_like(lay["B"])
    lay["C"] = torch.ones_like(lay["C"])
    y, s = ssd.oracle_ssd_fwd(*(lay[k] for k in workloads.SSD_KEYS), lib=lib)
    a = _np(lay)
    delta = float(np.logaddexp(0.0, a["dt_bias"][0]))
    xs = a["x"][0, :, 0, 0]
    S = scipy.signal.lfilter([delta], [1.0, -np.exp(delta * a["A"][0])], xs)
    return max(scaled_err(y[0, :, 0, 0], S + a["D"][0] * xs), scaled_err(s[0, 0, 0, 0], S[-1]))


def pin_steps(lib):
    lay = workloads.make_ssd(2, 13, 4, 3, 5, 2, torch.float32, seed=6)
    S0 = np.random.default_rng(6).standard_normal((2, 4, 3, 5))
    y, s = ssd.oracle_ssd_fwd(*(lay[k] for k in workloads.SSD_KEYS), state=S0, lib=lib)
    st = S0
    worst = 0.0
    for t in range(13):
        yt, st = ssd.oracle_ssd_step(lay["x"][:, t], lay["dt"][:, t], lay["B"][:, t], lay["C"][:, t],
                                     lay["dt_bias"], lay["A"], lay["D"], st, lib=lib)
        worst = max(worst, scaled_err(yt, y[:, t]))
    return max(worst, scaled_err(st, s))


def pin_resume(lib):
    lay = workloads.make_ssd(1, 20, 3, 4, 6, 1, torch.float32, seed=7)
    y, s = ssd.oracle_ssd_fwd(*(lay[k] for k in workloads.SSD_KEYS), lib=lib)
    worst = 0.0
    for k in (1, 5, 19):
        part = lambda sl, v: v[:, sl] if v.dim() >= 2 and v.shape[1] == 20 else v
        y1, s1 = ssd.oracle_ssd_fwd(*(part(slice(0, k), lay[q]) for q in workloads.SSD_KEYS), lib=lib)
        y2, s2 = ssd.oracle_ssd_fwd(*(part(slice(k, 20), lay[q]) for q in workloads.SSD_KEYS), state=s1, lib=lib)
        worst = max(worst, scaled_err(np.concatenate([y1, y2], 1), y), scaled_err(s2, s))
    return worst


def pin_packed(lib):
    """Packed documents (seq_idx) == each document run on its own from a zero
    state, the first one from the given state; y concatenated, the final state
    that of the last document. Documents of lengths 1, 5, 2, 9, 3, 4 over two
    batch rows with boundaries at different positions."""
    import workloads as W
    worst = 0.0
    L = 24
    lay = W.make_ssd(2, L, 3, 4, 5, 1, torch.float32, seed=8)
    S0 = np.random.default_rng(8).standard_normal((2, 3, 4, 5))
    ids = np.array([[0] * 1 + [1] * 5 + [2] * 2 + [3] * 9 + [4] * 3 + [5] * 4,
                    [7] * 6 + [3] * 1 + [9] * 12 + [2] * 5], dtype=np.int32)
    y, s = ssd.oracle_ssd_fwd(*(lay[k] for k in workloads.SSD_KEYS), state=S0, lib=lib, seq_idx=ids)
    for b in range(2):
        cuts = [0] + [t for t in range(1, L) if ids[b, t] != ids[b, t - 1]] + [L]
        for i in range(len(cuts) - 1):
            a0, a1 = cuts[i], cuts[i + 1]
            part = {k: (v[b:b + 1, a0:a1] if v.dim() >= 2 else v) for k, v in lay.items()}
            st = S0[b:b + 1] if i == 0 else None
            yd, sd = ssd.oracle_ssd_fwd(*(part[k] for k in workloads.SSD_KEYS), state=st, lib=lib)
            worst = max(worst, scaled_err(y[b:b + 1, a0:a1], yd))
            if i == len(cuts) - 2:
                worst = max(worst, scaled_err(s[b:b + 1], sd))
    return worst


PINS = [("dual", pin_dual), ("a_zero", pin_a_zero), ("no_step", pin_no_step), ("iir", pin_iir),
        ("steps", pin_steps), ("resume", pin_resume), ("packed", pin_packed)]


def run_all(lib=None):
    """{name: worst scaled error} of every pin."""
    return {name: fn(lib) for name, fn in PINS}
