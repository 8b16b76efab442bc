"""Checks that pin the fp64 oracle to something other than itself.

Each function takes an oracle library handle (so the same checks can be run
against deliberately broken copies of the oracle) and returns the largest
scaled error it saw; the caller compares it with the bound given next to each
check. Independent evaluations use numpy / scipy / torch library routines or
50-digit mpmath, never the oracle's code.

Sources of the special cases: the mixer steps of calm-mamba 0.1.4 PKG-INFO
("Mamba operator", steps 2, 4, 5, 6), and the closed forms the method admits
(A = 0 makes the recurrence a prefix sum; delta = 0 freezes the state; a
single state with constant delta is a first-order IIR filter; a very fast
decay makes it memoryless).
"""
import mpmath
import numpy as np
import scipy.signal
import scipy.special
import torch

import oracle

# bounds for the scaled error max|g-w| / max(|w|, rms(w))
FP64_BOUND = 1e-12


def scaled_err(got, want):
    g, w = np.asarray(got, np.float64).ravel(), np.asarray(want, np.float64).ravel()
    rms = np.sqrt(np.mean(w * w)) if w.size else 0.0
    scale = np.maximum(np.abs(w), rms)
    scale[scale == 0] = 1.0
    return float(np.max(np.abs(g - w) / scale)) if w.size else 0.0


def rand_inputs(seed, batch=2, seqlen=11, d_inner=5, d_state=4, d_conv=4, states=True):
    rng = np.random.default_rng(seed)
    inp = dict(
        x=rng.standard_normal((batch, seqlen, d_inner)),
        dt=0.1 * rng.standard_normal((batch, seqlen, d_inner)),
        z=rng.standard_normal((batch, seqlen, d_inner)),
        B=rng.standard_normal((batch, seqlen, d_state)),
        C=rng.standard_normal((batch, seqlen, d_state)),
        conv_w=rng.uniform(-0.5, 0.5, (d_inner, d_conv)),
        conv_b=0.1 * rng.standard_normal(d_inner),
        dt_bias=rng.uniform(-4.0, -1.0, d_inner),
        D=1.0 + 0.5 * rng.standard_normal(d_inner),
        A=-rng.uniform(0.5, 8.0, (d_inner, d_state)),
    )
    if states:
        inp["conv_state"] = rng.standard_normal((batch, d_inner, d_conv - 1))
        inp["ssm_state"] = rng.standard_normal((batch, d_inner, d_state))
    return inp


def run(lib, inp):
    return oracle.oracle_fwd(inp["x"], inp["dt"], inp["z"], inp["B"], inp["C"], inp["conv_w"], inp["conv_b"],
                             inp["dt_bias"], inp["D"], inp["A"], inp.get("conv_state"), inp.get("ssm_state"),
                             lib=lib)


def history(inp):
    """x with the conv state prepended along time: [batch, K-1+L, d_inner]."""
    b, _, d = inp["x"].shape
    k1 = inp["conv_w"].shape[1] - 1
    cs = inp.get("conv_state")
    pre = np.zeros((b, k1, d)) if cs is None else np.transpose(cs, (0, 2, 1))
    return np.concatenate([pre, inp["x"]], axis=1)


def conv_numpy(inp):
    """Pre-activation conv output u [batch, L, d] via numpy.correlate (cross-correlation,
    'valid' over the history-extended sequence: tap K-1 meets the newest x)."""
    xt = history(inp)
    b, L, d = inp["x"].shape
    u = np.empty((b, L, d))
    for bi in range(b):
        for di in range(d):
            u[bi, :, di] = np.correlate(xt[bi, :, di], inp["conv_w"][di], mode="valid") + inp["conv_b"][di]
    return u


def conv_torch(inp):
    """The same conv via torch.nn.functional.conv1d(groups=d) in float64 on the CPU."""
    xt = torch.from_numpy(history(inp)).permute(0, 2, 1)  # [b, d, K-1+L]
    w = torch.from_numpy(inp["conv_w"]).unsqueeze(1)  # [d, 1, K]
    u = torch.nn.functional.conv1d(xt, w, bias=torch.from_numpy(inp["conv_b"]), groups=w.shape[0])
    return u.permute(0, 2, 1).numpy()


def silu_np(u):
    return u * scipy.special.expit(u)


def softplus_np(v):
    return np.logaddexp(0.0, v)


def pin_conv_freeze(lib, seed=1):
    """delta == 0 (dt_bias = -1e4 makes softplus exactly 0 in float64): h stays at
    h0, so y = (C.h0 + D*xc) * SiLU(z) with xc = SiLU(conv) from numpy and torch.
    Bound FP64_BOUND."""
    inp = rand_inputs(seed, batch=2, seqlen=9, d_inner=6, d_state=5)
    inp["dt_bias"] = np.full_like(inp["dt_bias"], -1e4)
    y, cs, ss = run(lib, inp)
    errs = []
    for u in (conv_numpy(inp), conv_torch(inp)):
        xc = silu_np(u)
        readout = np.einsum("bln,bdn->bld", inp["C"], inp["ssm_state"])
        want = (readout + inp["D"][None, None, :] * xc) * silu_np(inp["z"])
        errs.append(scaled_err(y, want))
    errs.append(scaled_err(ss, inp["ssm_state"]))
    # final conv state = last K-1 entries of the history-extended x
    errs.append(float(np.max(np.abs(cs - np.transpose(history(inp)[:, -3:, :], (0, 2, 1))))))
    return max(errs)


def pin_prefix_sum(lib, seed=2):
    """A == 0: exp(delta*A) = 1, so h_t = h0 + cumsum_t(delta*B*xc) (numpy.cumsum),
    y = (C.h + D*xc) * SiLU(z), delta = logaddexp(0, dt + dt_bias). Bound FP64_BOUND."""
    inp = rand_inputs(seed, batch=2, seqlen=13, d_inner=4, d_state=3)
    inp["A"] = np.zeros_like(inp["A"])
    y, cs, ss = run(lib, inp)
    xc = silu_np(conv_numpy(inp))
    delta = softplus_np(inp["dt"] + inp["dt_bias"][None, None, :])
    inc = (delta * xc)[..., None] * inp["B"][:, :, None, :]  # [b, L, d, n]
    h = inp["ssm_state"][:, None, :, :] + np.cumsum(inc, axis=1)
    want = (np.einsum("bln,bldn->bld", inp["C"], h) + inp["D"] * xc) * silu_np(inp["z"])
    return max(scaled_err(y, want), scaled_err(ss, h[:, -1]))


def pin_iir(lib, seed=3):
    """d_state = 1, constant delta per channel (dt = 0), B = 1: h is the first-order
    IIR filter h_t = a*h_{t-1} + delta*xc_t with a = exp(delta*A), evaluated by
    scipy.signal.lfilter with its initial condition a*h0. Bound FP64_BOUND."""
    inp = rand_inputs(seed, batch=2, seqlen=17, d_inner=3, d_state=1)
    inp["dt"] = np.zeros_like(inp["dt"])
    inp["B"] = np.ones_like(inp["B"])
    y, cs, ss = run(lib, inp)
    xc = silu_np(conv_numpy(inp))
    delta = softplus_np(inp["dt_bias"])
    want = np.empty_like(y)
    hend = np.empty_like(ss)
    for b in range(y.shape[0]):
        for d in range(y.shape[2]):
            a = np.exp(delta[d] * inp["A"][d, 0])
            h, _ = scipy.signal.lfilter([delta[d]], [1.0, -a], xc[b, :, d], zi=[a * inp["ssm_state"][b, d, 0]])
            want[b, :, d] = (inp["C"][b, :, 0] * h + inp["D"][d] * xc[b, :, d]) * silu_np(inp["z"][b, :, d])
            hend[b, d, 0] = h[-1]
    return max(scaled_err(y, want), scaled_err(ss, hend))


def pin_memoryless(lib, seed=4):
    """A = -1e6 with dt = 0 makes exp(delta*A) underflow to exactly 0 (delta >=
    1e-3), so h_t = delta*B_t*xc_t and y = (delta*(C_t.B_t) + D)*xc*SiLU(z).
    Bound FP64_BOUND."""
    inp = rand_inputs(seed, batch=2, seqlen=10, d_inner=4, d_state=6)
    inp["A"] = np.full_like(inp["A"], -1e6)
    inp["dt"] = np.zeros_like(inp["dt"])
    inp["dt_bias"] = np.log(np.expm1(np.linspace(1e-3, 0.1, inp["dt_bias"].size)))
    y, cs, ss = run(lib, inp)
    xc = silu_np(conv_numpy(inp))
    delta = softplus_np(inp["dt_bias"])[None, None, :]
    cb = np.einsum("bln,bln->bl", inp["C"], inp["B"])[:, :, None]
    want = (delta * cb + inp["D"]) * xc * silu_np(inp["z"])
    hend = delta[0, 0][None, :, None] * xc[:, -1, :, None] * inp["B"][:, -1, None, :]
    return max(scaled_err(y, want), scaled_err(ss, hend))


def pin_brute_force(lib, seed=5, digits=50):
    """L <= 8: every output from the non-recursive sum
    h_t[n] = e^{A_n sum_{r<=t} delta_r} h0[n] + sum_{s<=t} e^{A_n sum_{s<r<=t} delta_r} delta_s B_s[n] xc_s,
    with conv, softplus and SiLU from their definitions, all in mpmath at
    `digits` digits. Bound 1e-14."""
    inp = rand_inputs(seed, batch=2, seqlen=7, d_inner=3, d_state=4)
    y, cs, ss = run(lib, inp)
    mp = mpmath.mp
    old = mp.dps
    mp.dps = digits
    try:
        mpf = mpmath.mpf
        b_, L, D_ = inp["x"].shape
        N = inp["B"].shape[2]
        want = np.empty_like(y)
        hend = np.empty_like(ss)
        for b in range(b_):
            for d in range(D_):
                hist = [mpf(float(v)) for v in inp["conv_state"][b, d]]
                xs = hist + [mpf(float(v)) for v in inp["x"][b, :, d]]
                xc, dl = [], []
                for t in range(L):
                    u = mpf(float(inp["conv_b"][d])) + sum(mpf(float(inp["conv_w"][d, k])) * xs[t + k]
                                                           for k in range(4))
                    xc.append(u / (1 + mpmath.exp(-u)))
                    v = mpf(float(inp["dt"][b, t, d])) + mpf(float(inp["dt_bias"][d]))
                    dl.append(mpmath.log(1 + mpmath.exp(v)))
                for t in range(L):
                    acc = mpf(0)
                    for n in range(N):
                        An = mpf(float(inp["A"][d, n]))
                        hn = mpmath.exp(An * sum(dl[: t + 1])) * mpf(float(inp["ssm_state"][b, d, n]))
                        for s in range(t + 1):
                            hn += (mpmath.exp(An * sum(dl[s + 1: t + 1])) * dl[s]
                                   * mpf(float(inp["B"][b, s, n])) * xc[s])
                        acc += mpf(float(inp["C"][b, t, n])) * hn
                        if t == L - 1:
                            hend[b, d, n] = float(hn)
                    zt = mpf(float(inp["z"][b, t, d]))
                    want[b, t, d] = float((acc + mpf(float(inp["D"][d])) * xc[t]) * zt / (1 + mpmath.exp(-zt)))
    finally:
        mp.dps = old
    return max(scaled_err(y, want), scaled_err(ss, hend))


def pin_step_chain(lib, seed=6):
    """oracle_step applied token by token reproduces oracle_fwd's outputs and final
    states (step is a separate implementation). Bound 1e-14 (the pages report
    1.6e-15 for the same check on Mamba-2 in float64)."""
    inp = rand_inputs(seed, batch=3, seqlen=12, d_inner=5, d_state=4)
    y, cs, ss = run(lib, inp)
    c, s = inp["conv_state"], inp["ssm_state"]
    ys = []
    for t in range(inp["x"].shape[1]):
        yt, c, s = oracle.oracle_step(inp["x"][:, t], inp["dt"][:, t], inp["z"][:, t], inp["B"][:, t],
                                      inp["C"][:, t], inp["conv_w"], inp["conv_b"], inp["dt_bias"], inp["D"],
                                      inp["A"], c, s, lib=lib)
        ys.append(yt)
    return max(scaled_err(np.stack(ys, 1), y), scaled_err(s, ss), float(np.max(np.abs(c - cs))))


def pin_resume(lib, seed=7):
    """fwd over x[:k] then fwd over x[k:] from the returned states equals fwd over x
    (k in 1, 2, 3, 4, L-1); conv state exactly. Bound 1e-14."""
    inp = rand_inputs(seed, batch=2, seqlen=10, d_inner=4, d_state=3)
    y, cs, ss = run(lib, inp)
    err = 0.0
    L = inp["x"].shape[1]
    for k in (1, 2, 3, 4, L - 1):
        a = dict(inp)
        bb = dict(inp)
        for key in ("x", "dt", "z", "B", "C"):
            a[key] = np.ascontiguousarray(inp[key][:, :k])
            bb[key] = np.ascontiguousarray(inp[key][:, k:])
        y1, c1, s1 = run(lib, a)
        bb["conv_state"], bb["ssm_state"] = c1, s1
        y2, c2, s2 = run(lib, bb)
        err = max(err, scaled_err(np.concatenate([y1, y2], 1), y), scaled_err(s2, ss),
                  float(np.max(np.abs(c2 - cs))))
    return err


def pin_linearity(lib, seed=8):
    """y - D*xc*SiLU(z) is linear in C, and the output is affine in h0:
    f(h1 + h2) - f(0) = (f(h1) - f(0)) + (f(h2) - f(0)). Bound 1e-12."""
    inp = rand_inputs(seed, batch=2, seqlen=9, d_inner=4, d_state=5)
    rng = np.random.default_rng(seed + 100)
    C1, C2 = rng.standard_normal(inp["C"].shape), rng.standard_normal(inp["C"].shape)
    y0 = run(lib, dict(inp, C=np.zeros_like(C1)))[0]  # = D*xc*SiLU(z)
    y1 = run(lib, dict(inp, C=C1))[0]
    y2 = run(lib, dict(inp, C=C2))[0]
    y12 = run(lib, dict(inp, C=C1 + C2))[0]
    e1 = scaled_err(y12 - y0, (y1 - y0) + (y2 - y0))
    h1, h2 = rng.standard_normal(inp["ssm_state"].shape), rng.standard_normal(inp["ssm_state"].shape)
    f0 = run(lib, dict(inp, ssm_state=np.zeros_like(h1)))
    f1 = run(lib, dict(inp, ssm_state=h1))
    f2 = run(lib, dict(inp, ssm_state=h2))
    f12 = run(lib, dict(inp, ssm_state=h1 + h2))
    e2 = scaled_err(f12[0] - f0[0], (f1[0] - f0[0]) + (f2[0] - f0[0]))
    e3 = scaled_err(f12[2] - f0[2], (f1[2] - f0[2]) + (f2[2] - f0[2]))
    # and the C-linear part is not identically zero (the check has teeth)
    assert np.max(np.abs(y1 - y0)) > 1e-3
    return max(e1, e2, e3)


def pin_causality(lib, seed=9):
    """Perturbing x at t0 leaves out[t < t0] bit-identical; permuting channels (with
    their parameters) or batch rows permutes the outputs exactly. Returns 0 or 1."""
    inp = rand_inputs(seed, batch=3, seqlen=12, d_inner=5, d_state=4)
    y = run(lib, inp)[0]
    bad = 0.0
    for t0 in (0, 1, 5, 11):
        p = dict(inp, x=inp["x"].copy())
        p["x"][:, t0, :] += 1.0
        yp = run(lib, p)[0]
        if not np.array_equal(yp[:, :t0], y[:, :t0]):
            bad = 1.0
        if np.array_equal(yp[:, t0], y[:, t0]):
            bad = 1.0  # the perturbation must reach its own timestep
    perm = np.array([3, 0, 4, 1, 2])
    q = dict(inp)
    for k in ("x", "dt", "z"):
        q[k] = np.ascontiguousarray(inp[k][:, :, perm])
    for k in ("conv_w", "conv_b", "dt_bias", "D", "A"):
        q[k] = np.ascontiguousarray(inp[k][perm])
    for k in ("conv_state", "ssm_state"):
        q[k] = np.ascontiguousarray(inp[k][:, perm])
    yq, cq, sq = run(lib, q)
    y0, c0, s0 = run(lib, inp)
    if not (np.array_equal(yq, y0[:, :, perm]) and np.array_equal(sq, s0[:, perm]) and np.array_equal(cq, c0[:, perm])):
        bad = 1.0
    bperm = np.array([2, 0, 1])
    r = {k: (np.ascontiguousarray(v[bperm]) if k in ("x", "dt", "z", "B", "C", "conv_state", "ssm_state") else v)
         for k, v in inp.items()}
    yr = run(lib, r)[0]
    if not np.array_equal(yr, y0[bperm]):
        bad = 1.0
    return bad


def run_seq(lib, inp, seq_idx):
    return oracle.oracle_fwd(inp["x"], inp["dt"], inp["z"], inp["B"], inp["C"], inp["conv_w"], inp["conv_b"],
                             inp["dt_bias"], inp["D"], inp["A"], inp.get("conv_state"), inp.get("ssm_state"),
                             lib=lib, seq_idx=seq_idx)


def seq_concat_err(lib, inp, ids):
    """Largest scaled error between the packed run over `ids` and running every
    document of every row on its own (the first from the given states, the
    others from zero states); conv state compared exactly (inf if not)."""
    import workloads
    y, cs, ss = run_seq(lib, inp, ids)
    err = 0.0
    for b in range(ids.shape[0]):
        for k, (s0, s1) in enumerate(workloads.segments(ids[b])):
            part = {key: np.ascontiguousarray(inp[key][b:b + 1, s0:s1]) for key in ("x", "dt", "z", "B", "C")}
            for key in ("conv_w", "conv_b", "dt_bias", "D", "A"):
                part[key] = inp[key]
            if k == 0:
                part["conv_state"] = inp["conv_state"][b:b + 1]
                part["ssm_state"] = inp["ssm_state"][b:b + 1]
            yp, cp, sp = run(lib, part)
            err = max(err, scaled_err(y[b:b + 1, s0:s1], yp))
        err = max(err, scaled_err(ss[b:b + 1], sp))
        if not np.array_equal(cs[b:b + 1], cp):
            err = np.inf
    return err


def pin_seq_concat(lib, seed=10):
    """Packed documents (seq_idx strict reset, niverel-mamba 0.1.0 PKG-INFO)
    equal each document run separately, on the nine structural cases that page
    certifies at L = 40 (blocks of 8) and one at L = 8192; a constant seq_idx
    equals no seq_idx bitwise. Bound 1e-12 (the page reports 4.4e-16)."""
    import workloads
    err = 0.0
    inp = rand_inputs(seed, batch=2, seqlen=40, d_inner=3, d_state=4)
    for i, case in enumerate(workloads.SEQ_CASES):
        err = max(err, seq_concat_err(lib, inp, workloads.make_seq_idx(case, 2, 40, edge=8, seed=seed + i)))
    long = rand_inputs(seed + 1, batch=2, seqlen=8192, d_inner=2, d_state=3)
    err = max(err, seq_concat_err(lib, long, workloads.make_seq_idx("misaligned_rows", 2, 8192, seed=seed)))
    same = run_seq(lib, inp, np.full((2, 40), 5, np.int32))
    plain = run(lib, inp)
    if not all(np.array_equal(a, b) for a, b in zip(same, plain)):
        err = np.inf
    return err


GRAD_INPUTS = ("x", "dt", "z", "B", "C", "conv_w", "conv_b", "dt_bias", "D", "A")


def pin_gradients(lib, seed=11):
    """oracle_bwd against central finite differences of L = sum(y * dy) from
    oracle_fwd, along a random direction for each input separately (with
    incoming states); relative error of the directional derivative. Bound 1e-7
    (step 1e-5: truncation ~1e-10, rounding ~1e-11)."""
    inp = rand_inputs(seed, batch=2, seqlen=9, d_inner=3, d_state=4)
    rng = np.random.default_rng(seed + 1)
    dy = rng.standard_normal(inp["x"].shape)
    g = oracle.oracle_bwd(*(inp[k] for k in GRAD_INPUTS), dy, inp["conv_state"], inp["ssm_state"], lib=lib)
    loss = lambda q: float(np.sum(run(lib, q)[0] * dy))
    err = 0.0
    eps = 1e-5
    for k in GRAD_INPUTS:
        V = rng.standard_normal(inp[k].shape)
        hi = dict(inp, **{k: inp[k] + eps * V})
        lo = dict(inp, **{k: inp[k] - eps * V})
        fd = (loss(hi) - loss(lo)) / (2 * eps)
        an = float(np.sum(g["d" + k] * V))
        err = max(err, abs(fd - an) / max(abs(fd), 1e-3))
    return err


def pin_xc_input(lib, seed=12):
    """oracle_fwd_xc (the scan from a given activated conv output) fed
    xc = SiLU(conv) computed here with numpy.correlate reproduces the pinned
    oracle_fwd's outputs and final SSM state (with incoming states): a dropped
    or misplaced term of its recurrence, readout, D skip or gate would not."""
    inp = rand_inputs(seed, batch=2, seqlen=13, d_inner=5, d_state=4)
    y, _, ss = run(lib, inp)
    xc = silu_np(conv_numpy(inp))
    y2, ss2 = oracle.oracle_fwd_xc(xc, inp["dt"], inp["z"], inp["B"], inp["C"], inp["dt_bias"], inp["D"], inp["A"],
                                   inp["ssm_state"], lib=lib)
    return max(scaled_err(y2, y), scaled_err(ss2, ss))


# (name, function, bound)
PINS = [
    ("conv_freeze", pin_conv_freeze, FP64_BOUND),
    ("prefix_sum", pin_prefix_sum, FP64_BOUND),
    ("iir", pin_iir, FP64_BOUND),
    ("memoryless", pin_memoryless, FP64_BOUND),
    ("brute_force", pin_brute_force, 1e-14),
    ("step_chain", pin_step_chain, 1e-14),
    ("resume", pin_resume, 1e-14),
    ("linearity", pin_linearity, 1e-12),
    ("causality", pin_causality, 0.5),
    ("seq_concat", pin_seq_concat, FP64_BOUND),
    ("gradients", pin_gradients, 1e-7),
    ("xc_input", pin_xc_input, FP64_BOUND),
]
