"""A second pin of the oracle's hand-written backward, independent of it: torch
autograd (float64, CPU) through the forward written directly with torch ops
(calm-mamba 0.1.4 PKG-INFO, "Mamba operator", steps 2, 4, 5, 6), with and
without incoming states, on a ragged shape."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests import tolerances as T

IO_KEYS = ("x", "dt", "z", "B", "C")
PARAM_KEYS = ("conv_w", "conv_b", "dt_bias", "D", "A")
NAMES = dict(dx="x", ddt="dt", dz="z", dB="B", dC="C", dconv_w="conv_w", dconv_b="conv_b", ddt_bias="dt_bias",
             dD="D", dA="A")


def autograd_grads(lay, dy, cs, ss):
    t = {k: v.double().clone().requires_grad_(True) for k, v in lay.items()}
    b, L, d = lay["x"].shape
    n = lay["B"].shape[2]
    hist = torch.zeros(b, 3, d, dtype=torch.float64) if cs is None else cs.double().transpose(1, 2)
    xpad = torch.cat([hist, t["x"]], 1)
    u = t["conv_b"] + sum(t["conv_w"][:, k] * xpad[:, k:k + L] for k in range(4))
    xc = u * torch.sigmoid(u)
    delta = torch.nn.functional.softplus(t["dt"] + t["dt_bias"])
    h = torch.zeros(b, d, n, dtype=torch.float64) if ss is None else ss.double()
    ys = []
    for i in range(L):
        decay = torch.exp(delta[:, i, :, None] * t["A"])
        h = decay * h + (delta[:, i] * xc[:, i])[:, :, None] * t["B"][:, i, None, :]
        ys.append((h * t["C"][:, i, None, :]).sum(-1) + t["D"] * xc[:, i])
    y = torch.stack(ys, 1) * (t["z"] * torch.sigmoid(t["z"]))
    (y * dy.double()).sum().backward()
    return {k: t[src].grad.numpy() for k, src in NAMES.items()}


@pytest.mark.parametrize("states", [False, True])
@pytest.mark.parametrize("d_state", [8, 16])
def test_oracle_bwd_equals_autograd(states, d_state):
    b, L, d = 2, 19, 5
    lay = workloads.make_layer(b, L, d, d_state, torch.float32, seed=40 + d_state)
    g = torch.Generator().manual_seed(41)
    dy = torch.randn(b, L, d, generator=g)
    cs = torch.randn(b, d, 3, generator=g) if states else None
    ss = torch.randn(b, d, d_state, generator=g) if states else None
    want = autograd_grads(lay, dy, cs, ss)
    got = oracle.oracle_bwd(*(lay[k] for k in IO_KEYS + PARAM_KEYS), dy, cs, ss)
    for k in NAMES:
        T.assert_close(got[k], want[k], 1e-12, "oracle vs autograd " + k)
