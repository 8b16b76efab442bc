"""The fp64 oracle against closed forms, library routines, 50-digit brute force
and invariants (CPU only)."""
import numpy as np
import pytest

import oracle
from tests import pins


@pytest.fixture(scope="module")
def lib():
    return oracle._load()


@pytest.mark.parametrize("name,fn,bound", pins.PINS, ids=[p[0] for p in pins.PINS])
def test_pin(lib, name, fn, bound):
    err = fn(lib)
    assert err <= bound, "%s: %.3e > %.1e" % (name, err, bound)


def test_conv_state_short_sequences(lib):
    """L < 3: the new conv state is the last 3 of (conv_state ++ x), exactly."""
    for L in (1, 2, 3):
        inp = pins.rand_inputs(11 + L, batch=2, seqlen=L, d_inner=3, d_state=2)
        _, cs, _ = pins.run(lib, inp)
        want = np.transpose(pins.history(inp)[:, -3:, :], (0, 2, 1))
        assert np.array_equal(cs, want)


def test_zero_states_equal_absent_states(lib):
    inp = pins.rand_inputs(21, states=False)
    y0, c0, s0 = pins.run(lib, inp)
    z = dict(inp, conv_state=np.zeros((2, 5, 3)), ssm_state=np.zeros((2, 5, 4)))
    y1, c1, s1 = pins.run(lib, z)
    assert np.array_equal(y0, y1) and np.array_equal(c0, c1) and np.array_equal(s0, s1)


def test_rejects_bad_dims(lib):
    inp = pins.rand_inputs(22)
    with pytest.raises(ValueError):
        oracle.oracle_fwd(inp["x"][:, :0], inp["dt"][:, :0], inp["z"][:, :0], inp["B"][:, :0], inp["C"][:, :0],
                          inp["conv_w"], inp["conv_b"], inp["dt_bias"], inp["D"], inp["A"], lib=lib)


def test_threads_do_not_change_results(lib):
    inp = pins.rand_inputs(23, batch=3, seqlen=20, d_inner=17, d_state=16)
    a = oracle.oracle_fwd(*[inp[k] for k in ("x", "dt", "z", "B", "C", "conv_w", "conv_b", "dt_bias", "D", "A")],
                          nthreads=1, lib=lib)
    b = oracle.oracle_fwd(*[inp[k] for k in ("x", "dt", "z", "B", "C", "conv_w", "conv_b", "dt_bias", "D", "A")],
                          nthreads=4, lib=lib)
    for u, v in zip(a, b):
        assert np.array_equal(u, v)
