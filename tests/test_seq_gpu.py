"""Packed documents (mamba_scan_fwd_seq) on the GPU against the fp64 oracle
with the same seq_idx: the nine structural cases that niverel-mamba 0.1.0
PKG-INFO ("seq_idx strict reset") certifies, on every kernel family that
supports resets, split and unsplit, with and without incoming states; a
constant seq_idx equals the plain call bitwise; workload 1 at full size and a
long packed sequence (L = 8192)."""
import sys

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


def check_seq(lay_cpu, ids, rtol, with_states, seed, what, **kw):
    lay = H.to_gpu(lay_cpu)
    cs = ss = None
    b, L, d = lay_cpu["x"].shape
    n = lay_cpu["B"].shape[2]
    if with_states:
        g = torch.Generator().manual_seed(seed)
        cs = torch.randn(b, d, 3, generator=g).cuda()
        ss = torch.randn(b, d, n, generator=g).cuda()
    sq = torch.from_numpy(ids).cuda()
    y, cso, sso = H.gpu_fwd(lay, cs, ss, seq_idx=sq, **kw)
    torch.cuda.synchronize()
    cpu = {k: v.detach().cpu() for k, v in lay.items()}
    import oracle
    yo, cso_o, sso_o = oracle.oracle_fwd(*(cpu[k] for k in H.IO_KEYS + H.PARAM_KEYS),
                                         None if cs is None else cs.cpu(), None if ss is None else ss.cpu(),
                                         seq_idx=ids)
    T.assert_close(y, yo, rtol, what + " y")
    T.assert_close(sso, sso_o, rtol, what + " ssm_state")
    T.assert_bitwise(cso, cso_o, what + " conv_state")


SHAPES = [
    # (kind, batch, seqlen, d_inner, d_state, dtype)
    ("default", 8, 300, 1536, 16, torch.bfloat16),  # row kernel, unsplit
    ("row", 2, 300, 96, 16, torch.float32),        # row kernel split into chunks of 80
    ("quad", 1, 1000, 100, 16, torch.bfloat16),    # quad kernel split into chunks of 80
    ("default", 3, 257, 70, 8, torch.float32),     # d_state 8: quad kernel
]


@pytest.mark.parametrize("case", workloads.SEQ_CASES)
@pytest.mark.parametrize("shape", SHAPES, ids=["%s-%d-%d-%d-%d" % s[:5] for s in SHAPES])
def test_seq_cases(case, shape):
    kind, b, L, d, n, dtype = shape
    kw = {} if kind == "default" else dict(testing_kind=kind)
    say("seq", case, shape)
    lay = workloads.make_layer(b, L, d, n, dtype, seed=L + d + n, dt_range=(1e-4, 1e-1))
    ids = workloads.make_seq_idx(case, b, L, edge=16, seed=L)
    check_seq(lay, ids, T.RTOL[dtype], with_states=(case in ("boundary_at_0", "misaligned_rows",
                                                              "nonzero_first_id", "many_short_docs")),
              seed=L, what="%s %s" % (case, shape), **kw)


@pytest.mark.parametrize("shape", SHAPES, ids=["%s-%d-%d-%d-%d" % s[:5] for s in SHAPES])
def test_constant_seq_idx_is_the_plain_call(shape):
    kind, b, L, d, n, dtype = shape
    kw = {} if kind == "default" else dict(testing_kind=kind)
    lay = H.to_gpu(workloads.make_layer(b, L, d, n, dtype, seed=3, dt_range=(1e-4, 1e-1)))
    g = torch.Generator().manual_seed(2)
    cs = torch.randn(b, d, 3, generator=g).cuda()
    ss = torch.randn(b, d, n, generator=g).cuda()
    y1, c1, s1 = H.gpu_fwd(lay, cs, ss, **kw)
    y2, c2, s2 = H.gpu_fwd(lay, cs, ss, seq_idx=torch.full((b, L), 4, dtype=torch.int32, device="cuda"), **kw)
    torch.cuda.synchronize()
    T.assert_bitwise(y2, y1, "y")
    T.assert_bitwise(s2, s1, "ssm_state")
    T.assert_bitwise(c2, c1, "conv_state")


def test_workload1_packed_documents():
    """Workload 1's shape (B8 L2048 D1536 N16 bf16) with per-row misaligned
    documents, in its timed launch configuration (row kernel, unsplit)."""
    cfg = workloads.WORKLOADS[1]
    lay = workloads.make_config(1)
    ids = workloads.make_seq_idx("misaligned_rows", cfg["batch"], cfg["seqlen"], seed=11)
    check_seq(lay, ids, T.RTOL[cfg["dtype"]], with_states=False, seed=0, what="workload 1 packed")


def test_long_packed_sequence():
    """L = 8192 of many short documents (the page's length), batch 1, d_inner 1536:
    the quad kernel split into chunks, with boundaries inside and across chunks."""
    lay = workloads.make_layer(1, 8192, 1536, 16, torch.bfloat16, seed=8192, dt_range=(1e-4, 1e-1))
    ids = workloads.make_seq_idx("many_short_docs", 1, 8192, seed=5)
    check_seq(lay, ids, T.RTOL[torch.bfloat16], with_states=True, seed=1, what="L=8192 packed")


def test_lane_kernel_refuses_documents():
    lay = H.to_gpu(workloads.make_layer(1, 64, 64, 16, torch.float32, seed=1))
    with pytest.raises(ms.MambaScanError) as e:
        H.gpu_fwd(lay, seq_idx=torch.zeros(1, 64, dtype=torch.int32, device="cuda"), testing_kind="lane")
    assert e.value.status == 2
