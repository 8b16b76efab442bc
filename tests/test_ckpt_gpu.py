"""Training prefill with checkpoints (mamba_scan_fwd_ckpt) and the backward from
them (mamba_scan_bwd_ckpt) on the GPU.

The checkpoint of stage s is the state before timestep 16 s, so it is pinned
by the oracle's final state over the first 16 s timesteps (a separate oracle
run on that prefix; stage 0 is the incoming state itself). The prefill's other
outputs follow the prefill's rule, the gradients the backward's (both against
the oracle), on ragged lengths, channel counts that leave a workgroup part
empty, and sequences the row kernel splits into chunks (the checkpoints of
later chunks then come from the carried summaries). At the measured layer
(8 x 2048 x 1536 bf16, one unsplit chunk) the forward's outputs equal the plain
prefill's, and the gradients the plain backward's, bit for bit.

Agreement rule: per element, |got - want| <= rtol * max(|want|, rms(want)),
rtol 1e-4 for float32 io and 2e-2 for bfloat16 io."""
import sys

import pytest
import torch

import selective_state_space_07_amd as ms
import workloads
from tests import harness as H
from tests import tolerances as T

pytestmark = pytest.mark.gpu

GRADS = ("dx", "ddt", "dz", "dB", "dC", "dconv_w", "dconv_b", "ddt_bias", "dD", "dA")


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def inputs(b, L, d, dtype, with_states, seed):
    lay_cpu = workloads.make_layer(b, L, d, 16, dtype, seed=seed)
    g = torch.Generator().manual_seed(seed + 1)
    dy = torch.randn(b, L, d, generator=g).to(dtype)
    cs = torch.randn(b, d, 3, generator=g) if with_states else None
    ss = torch.randn(b, d, 16, generator=g) if with_states else None
    return lay_cpu, dy, cs, ss


def prefix(lay_cpu, t):
    return {k: (v[:, :t].contiguous() if k in H.IO_KEYS else v) for k, v in lay_cpu.items()}


CASES = [
    # (batch, seqlen, d_inner, dtype, states)
    (2, 40, 64, torch.float32, True),      # one chunk, ragged last stage
    (1, 257, 20, torch.float32, True),     # 20 channels (a workgroup part empty), one step past 16 stages
    (2, 700, 96, torch.bfloat16, True),    # the row kernel splits the sequence (9 chunks of 80)
    (1, 4096, 32, torch.float32, False),   # 64 chunks of 64
]


@pytest.mark.parametrize("case", CASES, ids=["%d-%d-%d-%s-%s" % (c[0], c[1], c[2], str(c[3])[6:], c[4])
                                             for c in CASES])
def test_fwd_ckpt_and_bwd_from_it(case):
    b, L, d, dtype, st = case
    say("ckpt", case)
    lay_cpu, dy, cs, ss = inputs(b, L, d, dtype, st, seed=L + d)
    lay = H.to_gpu(lay_cpu)
    p = H.params_of(lay)
    csg = None if cs is None else cs.cuda()
    ssg = None if ss is None else ss.cuda()
    ck = ms.ckpt_like(lay["x"])
    y, cso, sso = ms.fwd(*(lay[k] for k in H.IO_KEYS), p, csg, ssg, ckpt=ck)
    torch.cuda.synchronize()
    yo, cso_o, sso_o = H.oracle_fwd(lay_cpu, cs, ss)
    T.assert_close(y, yo, T.RTOL[dtype], "%s y" % (case,))
    T.assert_close(sso, sso_o, T.RTOL[dtype], "%s ssm_state" % (case,))
    T.assert_bitwise(cso, torch.from_numpy(cso_o).float(), "%s conv_state" % (case,))
    # checkpoints: stage 0 is the incoming state; stage s the oracle's state after 16 s steps
    stages = (L + 15) // 16
    want0 = torch.zeros(b, d, 16) if ss is None else ss
    T.assert_bitwise(ck[:, 0].cpu(), want0, "%s ckpt stage 0" % (case,))
    for s in sorted({1, stages // 2, stages - 1} - {0}):
        _, _, h = H.oracle_fwd(prefix(lay_cpu, 16 * s), cs, ss)
        T.assert_close(ck[:, s], h, T.RTOL[dtype], "%s ckpt stage %d" % (case, s))
    # the backward from the checkpoints against the oracle's gradients
    got = ms.bwd(*(lay[k] for k in H.IO_KEYS), p, dy.cuda(), csg, ssg, ckpt=ck)
    torch.cuda.synchronize()
    import oracle
    want = oracle.oracle_bwd(*(lay_cpu[k] for k in H.IO_KEYS + H.PARAM_KEYS), dy, cs, ss)
    for k in GRADS:
        s_ = T.assert_close(got[k], want[k], T.RTOL[dtype], "%s %s" % (case, k))
        say("  %-8s max_scaled %.2e" % (k, s_["max_scaled"]))


def test_measured_layer_is_bitwise_the_plain_path():
    """8 x 2048 x 1536 bf16: the checkpointing prefill's outputs equal the plain
    prefill's, and the backward from its checkpoints the recomputing backward's,
    bit for bit; sampled checkpoints against the oracle."""
    say("ckpt layer 8x2048x1536 bf16")
    lay_cpu, dy, _, _ = inputs(8, 2048, 1536, torch.bfloat16, False, seed=23)
    lay = H.to_gpu(lay_cpu)
    p = H.params_of(lay)
    ck = ms.ckpt_like(lay["x"])
    y1, c1, s1 = ms.fwd(*(lay[k] for k in H.IO_KEYS), p, ckpt=ck)
    y0, c0, s0 = ms.fwd(*(lay[k] for k in H.IO_KEYS), p)
    dyg = dy.cuda()
    g1 = ms.bwd(*(lay[k] for k in H.IO_KEYS), p, dyg, ckpt=ck)
    g0 = ms.bwd(*(lay[k] for k in H.IO_KEYS), p, dyg)
    torch.cuda.synchronize()
    T.assert_bitwise(y1, y0, "y")
    T.assert_bitwise(c1, c0, "conv_state")
    T.assert_bitwise(s1, s0, "ssm_state")
    for k in GRADS:
        T.assert_bitwise(g1[k], g0[k], k)
    chans = workloads.sample_channels(1536, 24, seed=5)
    for s in (1, 64, 127):
        _, _, h = H.oracle_fwd(prefix(lay_cpu, 16 * s), channels=chans)
        T.assert_close(ck[:, s][:, chans], h, T.RTOL[torch.bfloat16], "ckpt stage %d" % s)


@pytest.mark.parametrize("L", [40, 700])
def test_ckpt_per_stage_descriptor_path_is_bitwise_the_same(L):
    """The testing entry point's force_wide takes the row kernel's per-stage-descriptor path
    (the one for chunks of 2 GiB or more) at any size: outputs, states and
    checkpoints equal the chunk-descriptor path's bit for bit, unsplit (L 40)
    and split into chunks (L 700)."""
    lay_cpu, _, cs, ss = inputs(2, L, 96, torch.bfloat16, True, seed=L)
    lay = H.to_gpu(lay_cpu)
    p = H.params_of(lay)
    outs = []
    for wide in (False, True):
        ck = ms.ckpt_like(lay["x"])
        y, c1, s1 = ms.fwd(*(lay[k] for k in H.IO_KEYS), p, cs.cuda(), ss.cuda(), ckpt=ck, testing_force_wide=wide)
        torch.cuda.synchronize()
        outs.append((y, c1, s1, ck))
    for a, b, what in zip(outs[0], outs[1], ("y", "conv_state", "ssm_state", "ckpt")):
        T.assert_bitwise(b, a, "%s L=%d" % (what, L))
