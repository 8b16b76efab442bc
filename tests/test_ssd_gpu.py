"""Mamba-2 SSD scan (mamba2_ssd_fwd) on the GPU against the pinned fp64 oracle:
float32 and bfloat16 io, d_state 64 and 128, one and two groups, ragged chunk
tails (L not a multiple of 256 or 64), L = 1, incoming states, the
Foundation-V3-like layer (24 heads of 64, d_state 128) at 8 x 2048 in full,
split/resume, in-place state and bitwise run-to-run determinism.

Agreement rule: the sealed rule of the Mamba-1 scan (per element,
|got - want| <= rtol * max(|want|, rms(want)), rtol 1e-4 for float32 io and
2e-2 for bfloat16 io) on y and on the final state."""
import sys

import pytest
import torch

import selective_state_space_07_amd as ms
import workloads
from oracle import ssd as ossd
from tests import tolerances as T

pytestmark = pytest.mark.gpu
K = workloads.SSD_KEYS


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def gpu(lay):
    return {k: v.cuda() for k, v in lay.items()}


def run(b, L, H, N, G, dtype, with_state, seed):
    lay = workloads.make_ssd(b, L, H, 64, N, G, dtype, seed=seed)
    s0 = torch.randn(b, H, 64, N, generator=torch.Generator().manual_seed(seed + 1)) if with_state else None
    g = gpu(lay)
    y, s = ms.ssd_fwd(*(g[k] for k in K), None if s0 is None else s0.cuda())
    torch.cuda.synchronize()
    yo, so = ossd.oracle_ssd_fwd(*(lay[k] for k in K), state=s0)
    return y, s, yo, so


SHAPES = [
    # (batch, seqlen, nheads, d_state, ngroups, dtype, state)
    (1, 256, 2, 64, 1, torch.float32, False),      # one full chunk
    (2, 300, 3, 128, 1, torch.bfloat16, True),     # ragged second chunk (44 steps)
    (1, 64, 4, 128, 2, torch.float32, True),       # two groups, one t-tile
    (2, 513, 6, 128, 1, torch.float32, True),      # three chunks, last one step long
    (1, 1, 1, 64, 1, torch.float32, True),         # one step
    (1, 190, 8, 64, 4, torch.bfloat16, False),     # ragged t-tiles, four groups
    (1, 2048, 24, 128, 1, torch.bfloat16, True),   # the layer's heads at L 2048
]


@pytest.mark.parametrize("shape", SHAPES, ids=["%d-%d-%d-%d-%d-%s-%s" % (s[0], s[1], s[2], s[3], s[4], str(s[5])[6:],
                                                                        s[6]) for s in SHAPES])
def test_ssd_matches_oracle(shape):
    b, L, H, N, G, dtype, st = shape
    say("ssd", shape)
    y, s, yo, so = run(b, L, H, N, G, dtype, st, seed=L + H + N)
    sy = T.assert_close(y, yo, T.RTOL[dtype], "%s y" % (shape,))
    ss = T.assert_close(s, so, T.RTOL[dtype], "%s state" % (shape,))
    say("  y max_scaled %.2e rel_l2 %.2e | state max_scaled %.2e" % (sy["max_scaled"], sy["rel_l2"], ss["max_scaled"]))


def test_ssd_full_layer():
    """8 x 2048 tokens, 24 heads of 64, d_state 128, bfloat16: every output."""
    say("ssd full 8x2048x24x64x128 bf16")
    y, s, yo, so = run(8, 2048, 24, 128, 1, torch.bfloat16, False, seed=31)
    sy = T.assert_close(y, yo, T.RTOL[torch.bfloat16], "full y")
    ss = T.assert_close(s, so, T.RTOL[torch.bfloat16], "full state")
    say("  y max_scaled %.2e | state max_scaled %.2e" % (sy["max_scaled"], ss["max_scaled"]))


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_ssd_resume_and_in_place_state(dtype):
    """fwd(x[:k]) then fwd(x[k:], state) agrees with fwd(x); the second call updates its state in place."""
    lay = gpu(workloads.make_ssd(2, 700, 4, 64, 128, 1, dtype, seed=41))
    y, s = ms.ssd_fwd(*(lay[k] for k in K))
    k = 333
    first = {q: (v[:, :k].contiguous() if v.dim() >= 3 else v) for q, v in lay.items()}
    second = {q: (v[:, k:].contiguous() if v.dim() >= 3 else v) for q, v in lay.items()}
    y1, s1 = ms.ssd_fwd(*(first[q] for q in K))
    y2, s2 = ms.ssd_fwd(*(second[q] for q in K), s1, state_out=s1)
    torch.cuda.synchronize()
    assert s2 is s1
    T.assert_close(torch.cat([y1, y2], 1), y, T.RTOL[dtype], "resumed y")
    T.assert_close(s2, s, T.RTOL[dtype], "resumed state")


def test_ssd_is_deterministic():
    lay = gpu(workloads.make_ssd(2, 600, 6, 64, 128, 1, torch.bfloat16, seed=43))
    y1, s1 = ms.ssd_fwd(*(lay[k] for k in K))
    ws = torch.full((ms.ssd_workspace_bytes(2, 600, 6, 64, 128, 1, torch.bfloat16),), 0x7F, dtype=torch.uint8,
                    device="cuda")
    y2, s2 = ms.ssd_fwd(*(lay[k] for k in K), workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2) and torch.equal(s1, s2)


@pytest.mark.parametrize("dtype,N,G", [(torch.float32, 64, 1), (torch.bfloat16, 128, 1), (torch.float32, 128, 2),
                                       (torch.bfloat16, 64, 4)])
def test_ssd_step_chain_matches_oracle(dtype, N, G):
    """Tokens one by one through mamba2_ssd_step (in place after the first) against
    oracle_ssd_step, and the chain's end against the GPU prefill of the same tokens."""
    b, L, H = 3, 20, 8
    lay = workloads.make_ssd(b, L, H, 64, N, G, dtype, seed=N + G)
    g = gpu(lay)
    s0 = torch.randn(b, H, 64, N, generator=torch.Generator().manual_seed(5))
    st = s0.cuda()
    st_o = s0.double().numpy()
    for t in range(L):
        y, st = ms.ssd_step(g["x"][:, t], g["dt"][:, t], g["B"][:, t], g["C"][:, t], g["dt_bias"], g["A"], g["D"], st,
                            inplace=t > 0)
        yo, st_o = ossd.oracle_ssd_step(lay["x"][:, t], lay["dt"][:, t], lay["B"][:, t], lay["C"][:, t],
                                        lay["dt_bias"], lay["A"], lay["D"], st_o)
        torch.cuda.synchronize()
        T.assert_close(y, yo, T.RTOL[dtype], "step %d y" % t)
    T.assert_close(st, st_o, T.RTOL[dtype], "step chain state")
    yf, sf = ms.ssd_fwd(*(g[k] for k in K), s0.cuda())
    torch.cuda.synchronize()
    T.assert_close(st, sf.cpu(), T.RTOL[dtype], "step chain vs prefill state")


def test_ssd_step_decode_batch_is_memory_bound_shape():
    """A decode-sized call (batch 256, 24 heads, d_state 128) against the oracle on sampled rows."""
    b, H, N = 256, 24, 128
    lay = workloads.make_ssd(b, 1, H, 64, N, 1, torch.bfloat16, seed=77)
    s0 = torch.randn(b, H, 64, N, generator=torch.Generator().manual_seed(78))
    g = gpu(lay)
    y, s1 = ms.ssd_step(g["x"][:, 0], g["dt"][:, 0], g["B"][:, 0], g["C"][:, 0], g["dt_bias"], g["A"], g["D"], s0.cuda())
    torch.cuda.synchronize()
    rows = [0, 1, 100, 255]
    yo, so = ossd.oracle_ssd_step(lay["x"][rows, 0], lay["dt"][rows, 0], lay["B"][rows, 0], lay["C"][rows, 0],
                                  lay["dt_bias"], lay["A"], lay["D"], s0[rows])
    T.assert_close(y[rows], yo, T.RTOL[torch.bfloat16], "decode y")
    T.assert_close(s1[rows], so, T.RTOL[torch.bfloat16], "decode state")


SEQ_SHAPES = [
    # (batch, seqlen, nheads, d_state, ngroups, dtype, edge)
    (2, 600, 4, 128, 1, torch.bfloat16, 64),     # three chunks, boundaries on t-tile edges
    (2, 530, 3, 64, 1, torch.float32, 256),      # boundaries on chunk edges
    (1, 300, 4, 128, 2, torch.float32, 16),      # off any tile edge
]


@pytest.mark.parametrize("case", workloads.SEQ_CASES)
@pytest.mark.parametrize("shape", SEQ_SHAPES, ids=["%d-%d-%d-%d-%d-%s-e%d" % (s[0], s[1], s[2], s[3], s[4],
                                                                             str(s[5])[6:], s[6]) for s in SEQ_SHAPES])
def test_ssd_packed_documents(case, shape):
    """The nine structural cases of niverel-mamba 0.1.0 PKG-INFO ("seq_idx strict
    reset") on the SSD scan, with an incoming state, against the oracle with the
    same seq_idx."""
    b, L, H, N, G, dtype, edge = shape
    say("ssd seq", case, shape)
    lay = workloads.make_ssd(b, L, H, 64, N, G, dtype, seed=L + H)
    ids = workloads.make_seq_idx(case, b, L, edge=edge, seed=L)
    s0 = torch.randn(b, H, 64, N, generator=torch.Generator().manual_seed(3))
    g = gpu(lay)
    y, s = ms.ssd_fwd(*(g[k] for k in K), s0.cuda(), seq_idx=torch.from_numpy(ids).cuda())
    torch.cuda.synchronize()
    yo, so = ossd.oracle_ssd_fwd(*(lay[k] for k in K), state=s0, seq_idx=ids)
    T.assert_close(y, yo, T.RTOL[dtype], "%s %s y" % (case, shape))
    T.assert_close(s, so, T.RTOL[dtype], "%s %s state" % (case, shape))


def test_ssd_constant_seq_idx_is_the_plain_call():
    lay = gpu(workloads.make_ssd(2, 700, 4, 64, 128, 1, torch.bfloat16, seed=5))
    s0 = torch.randn(2, 4, 64, 128, device="cuda")
    y1, s1 = ms.ssd_fwd(*(lay[k] for k in K), s0)
    y2, s2 = ms.ssd_fwd(*(lay[k] for k in K), s0, seq_idx=torch.full((2, 700), 3, dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    assert torch.equal(y1, y2) and torch.equal(s1, s2)


def test_ssd_packed_long_sequence():
    """L = 8192 (the length the pages certify at), documents of random lengths."""
    b, L, H, N = 1, 8192, 8, 128
    lay = workloads.make_ssd(b, L, H, 64, N, 1, torch.bfloat16, seed=88)
    rng = torch.Generator().manual_seed(89)
    lengths = torch.randint(1, 700, (40,), generator=rng)
    ids = torch.repeat_interleave(torch.arange(40), lengths)[:L]
    ids = torch.cat([ids, torch.full((L - ids.numel(),), 99)]).reshape(1, L).to(torch.int32)
    g = gpu(lay)
    y, s = ms.ssd_fwd(*(g[k] for k in K), seq_idx=ids.cuda())
    torch.cuda.synchronize()
    yo, so = ossd.oracle_ssd_fwd(*(lay[k] for k in K), seq_idx=ids.numpy())
    T.assert_close(y, yo, T.RTOL[torch.bfloat16], "L8192 y")
    T.assert_close(s, so, T.RTOL[torch.bfloat16], "L8192 state")
