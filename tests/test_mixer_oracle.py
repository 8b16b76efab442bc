"""Pins of the fp64 mixer-layer oracle (oracle/mixer.py), each independent of
how it composes its steps: a zero gate half gives exactly zero; zero C rows
reduce the layer to D*xc*SiLU(z) through out_proj, with xc from
numpy.correlate (catches a swap of the x/z halves or of the B/C rows, which
the incoming state would expose); zero dt rows make delta = softplus(dt_bias)
once (catches dt_bias applied twice or not at all); and token-by-token steps
reproduce the whole-sequence layer (the step is written separately)."""
import numpy as np
import torch

import oracle
import workloads
from oracle import mixer
from tests.pins import scaled_err


def layer(seed, batch=2, seqlen=9, d_model=6, d_inner=5, d_state=4, dt_rank=3):
    lay = workloads.make_mixer_layer(batch, seqlen, d_model, d_inner, d_state, dt_rank, torch.float32, seed=seed,
                                     conv_bias=0.3)
    lay = {k: v.double().numpy() for k, v in lay.items()}
    rng = np.random.default_rng(seed + 50)
    lay["conv_state"] = rng.standard_normal((batch, d_inner, 3))
    lay["ssm_state"] = rng.standard_normal((batch, d_inner, d_state))
    return lay


def run(lay):
    return mixer.mixer_fwd(lay["hidden"], *(lay[k] for k in workloads.MIXER_KEYS), lay["conv_state"],
                           lay["ssm_state"])


def xc_numpy(lay):
    """SiLU(conv) of x = hidden @ w_in[:d]^T with numpy.correlate per channel."""
    d = lay["w_in"].shape[0] // 2
    x = lay["hidden"] @ lay["w_in"][:d].T
    b, L, _ = x.shape
    xc = np.empty_like(x)
    for i in range(b):
        for c in range(d):
            seq = np.concatenate([lay["conv_state"][i, c], x[i, :, c]])
            pre = np.correlate(seq, lay["conv_w"][c], mode="valid") + lay["conv_b"][c]
            xc[i, :, c] = pre / (1.0 + np.exp(-pre))
    return x, xc


def test_zero_gate_half_gives_zero():
    lay = layer(1)
    d = lay["w_in"].shape[0] // 2
    lay["w_in"][d:] = 0.0
    out = run(lay)[0]
    assert np.array_equal(out, np.zeros_like(out))
    assert np.abs(run(layer(1))[0]).max() > 1e-3  # and not zero otherwise


def test_zero_C_rows_leave_the_skip_path():
    lay = layer(2)
    r = lay["w_dt"].shape[1]
    n = lay["A"].shape[1]
    lay["w_x"][r + n:] = 0.0
    d = lay["w_in"].shape[0] // 2
    _, xc = xc_numpy(lay)
    z = lay["hidden"] @ lay["w_in"][d:].T
    want = (lay["D"] * xc * (z / (1.0 + np.exp(-z)))) @ lay["w_out"].T
    assert scaled_err(run(lay)[0], want) < 1e-12


def test_zero_dt_rows_give_softplus_of_the_bias():
    lay = layer(3)
    r = lay["w_dt"].shape[1]
    n = lay["A"].shape[1]
    lay["w_x"][:r] = 0.0
    d = lay["w_in"].shape[0] // 2
    x, xc = xc_numpy(lay)
    z = lay["hidden"] @ lay["w_in"][d:].T
    B, C = xc @ lay["w_x"][r:r + n].T, xc @ lay["w_x"][r + n:].T
    y, cs, ss = oracle.oracle_fwd(x, np.zeros_like(x), z, B, C, lay["conv_w"], lay["conv_b"], lay["dt_bias"],
                                  lay["D"], lay["A"], lay["conv_state"], lay["ssm_state"])
    out, cs2, ss2 = run(lay)
    assert scaled_err(out, y @ lay["w_out"].T) < 1e-12 and scaled_err(ss2, ss) < 1e-12


def test_steps_reproduce_the_sequence():
    lay = layer(4)
    out, cs, ss = run(lay)
    c, s = lay["conv_state"], lay["ssm_state"]
    outs = []
    for t in range(lay["hidden"].shape[1]):
        o, c, s = mixer.mixer_step(lay["hidden"][:, t], *(lay[k] for k in workloads.MIXER_KEYS), c, s)
        outs.append(o)
    assert scaled_err(np.stack(outs, 1), out) < 1e-13
    assert scaled_err(s, ss) < 1e-13 and np.array_equal(c, cs)


def test_pins_catch_swapped_B_and_C(monkeypatch):
    good = mixer._split
    monkeypatch.setattr(mixer, "_split", lambda w, r, n: (lambda a, b, c: (a, c, b))(*good(w, r, n)))
    try:
        test_zero_C_rows_leave_the_skip_path()
    except AssertionError:
        return
    raise AssertionError("swapping B and C went unnoticed")
