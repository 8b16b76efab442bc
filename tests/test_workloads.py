"""The seeded generator: deterministic, and the recipe's values."""
import numpy as np
import torch

import workloads


def test_deterministic_and_seed_sensitive():
    a = workloads.make_layer(2, 8, 16, 4, torch.bfloat16, seed=3)
    b = workloads.make_layer(2, 8, 16, 4, torch.bfloat16, seed=3)
    c = workloads.make_layer(2, 8, 16, 4, torch.bfloat16, seed=4)
    for k in a:
        assert torch.equal(a[k], b[k])
    assert not torch.equal(a["x"], c["x"])


def test_recipe_values():
    lay = workloads.make_config(0)
    cfg = workloads.WORKLOADS[0]
    assert lay["x"].shape == (cfg["batch"], cfg["seqlen"], cfg["d_inner"]) and lay["x"].dtype == torch.float32
    n = torch.arange(1, cfg["d_state"] + 1, dtype=torch.float32)
    assert torch.equal(lay["A"], -n.expand(cfg["d_inner"], -1))  # -exp(log(n+1)) is exact in float32
    assert torch.equal(lay["D"], torch.ones(cfg["d_inner"]))
    assert torch.equal(lay["conv_b"], torch.zeros(cfg["d_inner"]))
    assert lay["conv_w"].abs().max() <= 0.5
    sp = torch.nn.functional.softplus(lay["dt_bias"].double())
    assert sp.min() >= 1e-3 * 0.999 and sp.max() <= 0.1 * 1.001
    assert abs(float(lay["dt"].double().std()) - 0.1) < 0.01


def test_bf16_values_are_rounded_once():
    lay = workloads.make_layer(1, 4, 8, 4, torch.bfloat16, seed=1)
    assert lay["x"].dtype == torch.bfloat16 and lay["A"].dtype == torch.float32
    # upcast is exact: float32 -> bfloat16 of an upcast value changes nothing
    assert torch.equal(lay["x"].float().to(torch.bfloat16), lay["x"])


def test_long_config_dt_range():
    # workload 3 draws dt_bias from log-uniform [1e-4, 1e-1] (small shape, same recipe)
    lay = workloads.make_layer(1, 4, 4096, 16, torch.bfloat16, seed=7003, dt_range=(1e-4, 1e-1))
    sp = torch.nn.functional.softplus(lay["dt_bias"].double())
    assert sp.min() < 2e-4 and sp.max() > 5e-2


def test_decode_layers_independent():
    layers = workloads.make_decode_layers(layers=3, batch=4, prefill_len=5, d_inner=8)
    assert len(layers) == 3
    assert layers[0]["prefill"]["x"].shape == (4, 5, 8) and layers[0]["token"]["x"].shape == (4, 8)
    assert not torch.equal(layers[0]["params"]["conv_w"], layers[1]["params"]["conv_w"])


def test_sample_channels():
    idx = workloads.sample_channels(1536, 64, seed=1)
    assert idx[0] == 0 and idx[-1] == 1535 and len(set(idx.tolist())) == len(idx)
    assert np.all(np.diff(idx) > 0)
