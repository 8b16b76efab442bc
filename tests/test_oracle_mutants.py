"""The pins have teeth: each plausible mistake, planted in a copy of the
oracle's C source and compiled on the CPU, must make at least one pin fail.
Also the harness's negative control: inputs with the selectivity removed
(dt, B, C replaced by their time means) must fail the parity rule against
the true oracle output."""
import os

import numpy as np
import pytest
import torch

import oracle
import oracle.build as obuild
from tests import pins, tolerances

# (name, exact text in mamba_oracle.c's oracle_fwd/oracle_step, replacement)
MUTANTS = [
    ("drop_D_skip", "const double yv = acc + Dskip[d] * xc;", "const double yv = acc;"),
    ("zoh_instead_of_euler", "h[n] = exp(delta * A[d * N + n]) * h[n] + delta * Bt[n] * xc;",
     "h[n] = exp(delta * A[d * N + n]) * h[n] + (exp(delta * A[d * N + n]) - 1.0) / A[d * N + n] * Bt[n] * xc;"),
    ("drop_decay", "h[n] = exp(delta * A[d * N + n]) * h[n] + delta * Bt[n] * xc;",
     "h[n] = h[n] + delta * Bt[n] * xc;"),
    ("decay_sign", "h[n] = exp(delta * A[d * N + n]) * h[n] + delta * Bt[n] * xc;",
     "h[n] = exp(-delta * A[d * N + n]) * h[n] + delta * Bt[n] * xc;"),
    ("readout_uses_B", "acc += Ct[n] * h[n];", "acc += Bt[n] * h[n];"),
    ("conv_flipped", "u += conv_w[d * K + k] * win[k];", "u += conv_w[d * K + (K - 1 - k)] * win[k];"),
    ("conv_bias_dropped", "double u = conv_b[d];", "double u = 0.0;"),
    ("conv_state_reversed", "hist[j] = conv_state_in ? conv_state_in[(b * D + d) * H + j] : 0.0;",
     "hist[j] = conv_state_in ? conv_state_in[(b * D + d) * H + (H - 1 - j)] : 0.0;"),
    ("dt_bias_sign", "softplus(dt[e] + dt_bias[d])", "softplus(dt[e] - dt_bias[d])"),
    ("no_softplus", "const double delta = softplus(dt[e] + dt_bias[d]);",
     "const double delta = dt[e] + dt_bias[d];"),
    ("gate_dropped", "y[e] = yv * silu(z[e]);", "y[e] = yv;"),
    ("readout_before_update", "h[n] = exp(delta * A[d * N + n]) * h[n] + delta * Bt[n] * xc;\n              acc += Ct[n] * h[n];",
     "acc += Ct[n] * h[n];\n              h[n] = exp(delta * A[d * N + n]) * h[n] + delta * Bt[n] * xc;"),
    ("ssm_state_not_loaded", "h[n] = ssm_state_in ? ssm_state_in[(b * D + d) * N + n] : 0.0;", "h[n] = 0.0;"),
    ("step_conv_shift_wrong", "shifted[k] = cs[k + 1];", "shifted[k] = cs[k];"),
    ("step_gate_on_x", "y[e] = yv * (z[e] / (1.0 + exp(-z[e])));", "y[e] = yv * (x[e] / (1.0 + exp(-x[e])));"),
    ("seq_keeps_conv_history", "for (int64_t j = 0; j < H; ++j) hist[j] = 0.0;\n", "\n"),
    ("seq_keeps_ssm_state", "for (int64_t n = 0; n < N; ++n) h[n] = 0.0;\n            }", "\n            }"),
    ("seq_reset_one_late", "seq_idx[b * L + t] != seq_idx[b * L + t - 1]",
     "t >= 2 && seq_idx[b * L + t - 1] != seq_idx[b * L + t - 2]"),
    ("seq_no_reset", "if (seq_idx && t > 0 &&", "if (0 && seq_idx && t > 0 &&"),
    ("bwd_state_grad_not_decayed", "dh[n] *= a;", "dh[n] *= 1.0;"),
    ("bwd_conv_transpose_shifted", "const int64_t p = t - H + k;", "const int64_t p = t - k;"),
    ("bwd_dA_uses_new_state", "pA[d * N + n] += dh[n] * delta * a * hprev[n];",
     "pA[d * N + n] += dh[n] * delta * a * h[n];"),
    ("bwd_softplus_grad_dropped", "const double dv = ddelta * sigm(v);", "const double dv = ddelta;"),
    ("bwd_gate_grad_wrong", "dz[e] = dy[e] * yraw * dsilu(z[e]);", "dz[e] = dy[e] * yraw * sigm(z[e]);"),
    ("xc_input_drops_D_skip", "y[e] = (acc + Dskip[d] * xc[e]) * silu(z[e]);", "y[e] = acc * silu(z[e]);"),
    ("xc_input_state_not_loaded", "h[n] = h0 ? h0[n] : 0.0;", "h[n] = 0.0;"),
    ("xc_input_dt_bias_sign", "const double pre = dt[e] + dt_bias[d];", "const double pre = dt[e] - dt_bias[d];"),
    ("xc_input_B_index", "delta * Bm[(b * L + t) * N + n] * xc[e];", "delta * Bm[(b * L + t) * N] * xc[e];"),
]


@pytest.fixture(scope="module")
def source():
    with open(obuild.SRC) as f:
        return f.read()


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, source, name, old, new):
    assert source.count(old) == 1, "anchor for %s not found exactly once in the oracle source" % name
    src = tmp_path / ("oracle_%s.c" % name)
    src.write_text(source.replace(old, new))
    so = obuild.build(src=str(src), out=str(tmp_path / ("lib_%s.so" % name)))
    lib = oracle.load_library(so)
    failed = []
    for pname, fn, bound in pins.PINS:
        try:
            err = fn(lib)
        except (AssertionError, ValueError, FloatingPointError):
            err = np.inf
        if not err <= bound:
            failed.append(pname)
    assert failed, "mutant %s passed every pin" % name


def test_negative_control_kill_selectivity():
    """Removing the input dependence of dt, B, C (time means) must fail the rule."""
    inp = pins.rand_inputs(31, batch=2, seqlen=64, d_inner=16, d_state=8)
    lib = oracle._load()
    y, _, _ = pins.run(lib, inp)
    k = dict(inp)
    for key in ("dt", "B", "C"):
        k[key] = np.broadcast_to(inp[key].mean(axis=1, keepdims=True), inp[key].shape).copy()
    yk, _, _ = pins.run(lib, k)
    ok, s = tolerances.within(yk, y, tolerances.RTOL[torch.bfloat16])
    assert not ok, s
    assert s["cosine"] < 0.99


def test_rule_accepts_bf16_rounding_and_rejects_small_errors():
    rng = np.random.default_rng(5)
    w = rng.standard_normal(10000)
    g_bf16 = torch.from_numpy(w).to(torch.bfloat16).double().numpy()
    assert tolerances.within(g_bf16, w, tolerances.RTOL[torch.bfloat16])[0]
    assert not tolerances.within(g_bf16, w, tolerances.RTOL[torch.float32])[0]
    g = w.copy()
    g[17] += 0.05 * max(abs(w[17]), 1.0)
    assert not tolerances.within(g, w, tolerances.RTOL[torch.bfloat16])[0]
    g = w.copy()
    g[3] = np.nan
    assert not tolerances.within(g, w, 1.0)[0]
