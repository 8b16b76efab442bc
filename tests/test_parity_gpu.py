"""HIP path (through the C ABI) against the fp64 oracle on the same seeded
inputs: the five workloads at full size, ragged shapes spanning several waves,
chunks and a ragged tail, both d_state values and both io dtypes."""
import sys

import numpy as np
import pytest
import torch

import selective_state_space_07_amd as ms
import workloads
from tests import harness as H
from tests import tolerances as T

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def check_fwd(layer_cpu, rtol, channels=None, with_states=False, seed=0, what=""):
    layer = H.to_gpu(layer_cpu)
    cs = ss = None
    if with_states:
        g = torch.Generator().manual_seed(seed)
        bsz, d = layer_cpu["x"].shape[0], layer_cpu["x"].shape[2]
        n = layer_cpu["B"].shape[2]
        cs = torch.randn(bsz, d, 3, generator=g).cuda()
        ss = torch.randn(bsz, d, n, generator=g).cuda()
    y, cso, sso = H.gpu_fwd(layer, cs, ss)
    torch.cuda.synchronize()
    yo, cso_o, sso_o = H.oracle_fwd(layer, cs, ss, channels=channels)
    s1 = T.assert_close(H.cols(y, channels, 2), yo, rtol, what + " y")
    s2 = T.assert_close(H.cols(sso, channels, 1), sso_o, rtol, what + " ssm_state")
    T.assert_bitwise(H.cols(cso, channels, 1), cso_o, what + " conv_state")
    return s1, s2


@pytest.mark.parametrize("index", [0, 1, 2])
def test_workload_full(index):
    cfg = workloads.WORKLOADS[index]
    say("workload", index, cfg["name"])
    s1, s2 = check_fwd(workloads.make_config(index), T.RTOL[cfg["dtype"]], what=cfg["name"])
    say("  y", s1, "\n  h", s2)


def test_workload_long_sampled():
    """Workload 3 at full size (batch 1, L 65536, d 1536) in its timed launch
    configuration; the oracle runs on 48 sampled channels over the whole sequence."""
    cfg = workloads.WORKLOADS[3]
    say("workload 3", cfg["name"])
    ch = workloads.sample_channels(cfg["d_inner"], 48, seed=3)
    s1, s2 = check_fwd(workloads.make_config(3), T.RTOL[cfg["dtype"]], channels=ch, what=cfg["name"])
    say("  y", s1, "\n  h", s2)


def test_workload_decode_sampled():
    """Workload 4 at full size: 24 layers of (GPU prefill of 128 tokens -> GPU step);
    the oracle runs prefill + step from its own states on 32 sampled channels per
    layer. The step kernel is also checked alone, fed the oracle's states."""
    cfg = workloads.WORKLOADS[4]
    rtol = T.RTOL[cfg["dtype"]]
    layers = workloads.make_decode_layers()
    ch = workloads.sample_channels(cfg["d_inner"], 32, seed=4)
    for li, lay in enumerate(layers):
        say("decode layer", li)
        pre = H.to_gpu(dict(lay["prefill"], **lay["params"]))
        params = H.params_of(pre)
        _, cs, ss = H.gpu_fwd(pre)
        tok = H.to_gpu(lay["token"])
        y, cs2, ss2 = H.gpu_step(tok, params, cs, ss)
        torch.cuda.synchronize()
        # oracle: prefill then step from its own states, on the sampled channels
        _, cso, sso = H.oracle_fwd(pre, channels=ch)
        yo, cs2o, ss2o = H.oracle_step(lay["token"], lay["params"], torch.from_numpy(cso),
                                       torch.from_numpy(sso), channels=ch, states_sliced=True)
        T.assert_close(H.cols(y, ch, 1), yo, rtol, "layer %d step y" % li)
        T.assert_close(H.cols(ss2, ch, 1), ss2o, rtol, "layer %d step ssm_state" % li)
        T.assert_bitwise(H.cols(cs2, ch, 1), cs2o, "layer %d step conv_state" % li)
        if li < 3:  # step alone from the oracle's (float32-rounded) states, every channel
            _, cs_o, ss_o = H.oracle_fwd(pre)
            cs_in = torch.from_numpy(cs_o).float().cuda()
            ss_in = torch.from_numpy(ss_o).float().cuda()
            y1, c1, s1 = H.gpu_step(tok, params, cs_in, ss_in)
            torch.cuda.synchronize()
            yo1, co1, so1 = H.oracle_step(lay["token"], lay["params"], cs_in, ss_in)
            T.assert_close(y1, yo1, rtol, "layer %d step-alone y" % li)
            T.assert_close(s1, so1, rtol, "layer %d step-alone ssm_state" % li)
            T.assert_bitwise(c1, co1, "layer %d step-alone conv_state" % li)


RAGGED = [
    # (batch, seqlen, d_inner, d_state, dtype)
    (1, 1, 1, 16, torch.float32),
    (2, 2, 65, 16, torch.float32),
    (1, 3, 100, 8, torch.bfloat16),
    (3, 5, 64, 8, torch.float32),
    (2, 63, 129, 16, torch.bfloat16),
    (1, 127, 200, 16, torch.float32),
    (1, 1000, 100, 16, torch.float32),   # split into chunks, ragged last chunk
    (2, 1037, 70, 8, torch.bfloat16),    # split, odd length
    (1, 4099, 64, 16, torch.bfloat16),   # many chunks
    (4, 200, 1536, 16, torch.bfloat16),
]


@pytest.mark.parametrize("shape", RAGGED, ids=[str(r[:4]) + str(r[4]).split(".")[-1] for r in RAGGED])
@pytest.mark.parametrize("with_states", [False, True])
def test_ragged(shape, with_states):
    b, L, d, n, dtype = shape
    say("ragged", shape, with_states, "workspace", ms.workspace_bytes(b, L, d, n, dtype))
    lay = workloads.make_layer(b, L, d, n, dtype, seed=hash(shape) % 1000, dt_range=(1e-4, 1e-1))
    check_fwd(lay, T.RTOL[dtype], with_states=with_states, seed=L, what=str(shape))


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("n", [8, 16])
def test_step_matches_oracle(dtype, n):
    lay = workloads.make_layer(5, 1, 300, n, dtype, seed=40 + n)
    tok = {k: lay[k][:, 0].contiguous() for k in H.IO_KEYS}
    params = {k: lay[k] for k in H.PARAM_KEYS}
    g = torch.Generator().manual_seed(n)
    cs, ss = torch.randn(5, 300, 3, generator=g), torch.randn(5, 300, n, generator=g)
    y, c2, s2 = H.gpu_step(H.to_gpu(tok), H.params_of(H.to_gpu(params)), cs.cuda(), ss.cuda())
    torch.cuda.synchronize()
    yo, co, so = H.oracle_step(tok, params, cs, ss)
    T.assert_close(y, yo, T.RTOL[dtype], "step y")
    T.assert_close(s2, so, T.RTOL[dtype], "step ssm_state")
    T.assert_bitwise(c2, co, "step conv_state")


KIND_SHAPES = [
    # (batch, seqlen, d_inner, d_state, dtype)
    (2, 300, 96, 16, torch.float32),      # row kernel split into 4 chunks, ragged last one
    (1, 1000, 100, 16, torch.bfloat16),   # ragged channel group, many chunks
    (3, 257, 70, 8, torch.float32),       # d_state 8 (the row kernel does not apply)
    (8, 300, 1536, 16, torch.bfloat16),   # row kernel unsplit, XCD-mapped grid
]


@pytest.mark.parametrize("kind", ["row", "quad", "lane"])
@pytest.mark.parametrize("shape", KIND_SHAPES, ids=[str(r[:4]) + str(r[4]).split(".")[-1] for r in KIND_SHAPES])
def test_forced_kernel_family(kind, shape, monkeypatch):
    """Every prefill kernel family, forced through the MSCAN_FWD_KIND knob, on
    shapes that the default plan sends elsewhere (so each family's split and
    unsplit paths run), with incoming states."""
    b, L, d, n, dtype = shape
    if kind == "row" and n != 16:
        pytest.skip("the row kernel serves d_state 16 only")
    monkeypatch.setenv("MSCAN_FWD_KIND", kind)
    say("forced", kind, shape, "workspace", ms.workspace_bytes(b, L, d, n, dtype))
    lay = workloads.make_layer(b, L, d, n, dtype, seed=L + d, dt_range=(1e-4, 1e-1))
    check_fwd(lay, T.RTOL[dtype], with_states=True, seed=L, what="%s %s" % (kind, shape))


@pytest.mark.parametrize("shape", [(8, 300, 1536, 16, torch.bfloat16), (2, 300, 96, 16, torch.float32)])
def test_row_wide_path_bitwise(shape, monkeypatch):
    """The row kernel's per-stage-descriptor path (taken when a chunk spans
    2 GiB or more) gives bit-identical results to the chunk-wide one."""
    b, L, d, n, dtype = shape
    monkeypatch.setenv("MSCAN_FWD_KIND", "row")
    lay = H.to_gpu(workloads.make_layer(b, L, d, n, dtype, seed=5, dt_range=(1e-4, 1e-1)))
    g = torch.Generator().manual_seed(1)
    cs = torch.randn(b, d, 3, generator=g).cuda()
    ss = torch.randn(b, d, n, generator=g).cuda()
    y1, c1, s1 = H.gpu_fwd(lay, cs, ss)
    monkeypatch.setenv("MSCAN_ROW_FORCE_WIDE", "1")
    y2, c2, s2 = H.gpu_fwd(lay, cs, ss)
    torch.cuda.synchronize()
    T.assert_bitwise(y2, y1, "wide y")
    T.assert_bitwise(s2, s1, "wide ssm_state")
    T.assert_bitwise(c2, c1, "wide conv_state")
