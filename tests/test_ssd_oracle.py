"""The Mamba-2 SSD oracle against its pins (tests/ssd_pins.py), and the pins'
teeth: each plausible mistake, planted in a copy of mamba2_oracle.c and
compiled on the CPU, must make at least one pin fail."""
import pytest

import oracle.build as obuild
from oracle import ssd
from tests import ssd_pins


@pytest.mark.parametrize("name,fn", ssd_pins.PINS, ids=[p[0] for p in ssd_pins.PINS])
def test_ssd_oracle_pin(name, fn):
    err = fn(None)
    assert err <= ssd_pins.PIN_TOL, "%s: scaled error %.3e" % (name, err)


# (name, exact text in mamba2_oracle.c, replacement)
MUTANTS = [
    ("decay_sign", "const double decay = exp(delta * A[h]);", "const double decay = exp(-delta * A[h]);"),
    ("drop_D_skip", "yt[p] = acc + Dskip[h] * xt[p];", "yt[p] = acc;"),
    ("no_softplus", "const double delta = softplus(dt[(b * seqlen + t) * nheads + h] + dt_bias[h]);",
     "const double delta = dt[(b * seqlen + t) * nheads + h] + dt_bias[h];"),
    ("input_without_delta", "Sp[n] = decay * Sp[n] + delta * xt[p] * Bt[n];", "Sp[n] = decay * Sp[n] + xt[p] * Bt[n];"),
    ("readout_uses_B", "acc += Ct[n] * Sp[n];", "acc += Bt[n] * Sp[n];"),
    ("readout_before_update", "Sp[n] = decay * Sp[n] + delta * xt[p] * Bt[n];\n            acc += Ct[n] * Sp[n];",
     "acc += Ct[n] * Sp[n];\n            Sp[n] = decay * Sp[n] + delta * xt[p] * Bt[n];"),
    ("group_index_wrong", "const int64_t g = h / heads_per_group;", "const int64_t g = h % ngroups;"),
    ("state_not_loaded", "for (int64_t i = 0; i < PN; ++i) S[i] = s0 ? s0[i] : 0.0;",
     "for (int64_t i = 0; i < PN; ++i) S[i] = 0.0;"),
    ("dt_bias_sign", "dt[(b * seqlen + t) * nheads + h] + dt_bias[h]", "dt[(b * seqlen + t) * nheads + h] - dt_bias[h]"),
    ("step_decay_dropped", "const double s_new = keep * state_in[base + n] + step * Bv[n] * xv;",
     "const double s_new = state_in[base + n] + step * Bv[n] * xv;"),
    ("seq_no_reset", "if (seq_idx && t > 0 &&", "if (0 && seq_idx && t > 0 &&"),
    ("seq_reset_one_late", "seq_idx[b * seqlen + t] != seq_idx[b * seqlen + t - 1]",
     "t >= 2 && seq_idx[b * seqlen + t - 1] != seq_idx[b * seqlen + t - 2]"),
    ("step_group_wrong", "const double* Bv = Bm + (b * ngroups + h / per_group) * d_state;",
     "const double* Bv = Bm + (b * ngroups + h % ngroups) * d_state;"),
]


@pytest.fixture(scope="module")
def source():
    with open(obuild.SSD_SRC) as f:
        return f.read()


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_ssd_mutant_is_caught(tmp_path, source, name, old, new):
    assert source.count(old) == 1, "anchor for %s not found exactly once" % name
    src = tmp_path / ("m_%s.c" % name)
    src.write_text(source.replace(old, new))
    lib = ssd.load_library(obuild.build(str(src), str(tmp_path / ("m_%s.so" % name))))
    errs = ssd_pins.run_all(lib)
    assert max(errs.values()) > 1e-6, "mutant %s passes every pin: %s" % (name, errs)
