"""Backward of the prefill at the size limit: batch 1, seqlen 2047, d_inner
2^20, d_state 16, bfloat16 io (batch * seqlen * d_inner = 2,146,435,072, just
under 2^31): every io tensor spans 4 GiB and the recomputing backward keeps
8.6 GB of its own checkpoints and 17 GB of dB / dC partials.

- The per-channel gradients (dx, ddt, dz, dconv_w, dconv_b, ddt_bias, dD, dA)
  of 24 channels (workgroup edges, both ends of d_inner, random ones) against
  the oracle run on those channels alone.
- The checkpointing pair (mamba_scan_fwd_ckpt writing 8.6 GB of states, then
  mamba_scan_bwd_ckpt) gives the same gradients bit for bit.
- dB and dC sum over all channels, so no channel subset pins them; they are
  checked by linearity in the channels instead: the full call's dB / dC equal
  the sum of those of two calls on the lower and upper halves of the channels
  (summed in another order, so to a relative 1e-3 of the scale below).

Inputs: parameters follow the shared recipe (workloads.make_layer, d_inner
2^20); x, z, B, C, dy ~ N(0, 1) and dt ~ 0.1 N(0, 1), drawn on the device from a
seeded generator and rounded to bfloat16.

Agreement rule: per element, |got - want| <= rtol * max(|want|, rms(want)),
rtol 2e-2 against the oracle."""
import sys

import numpy as np
import pytest
import torch

import oracle
import selective_state_space_07_amd as ms
import workloads
from tests import harness as H
from tests import tolerances as T

pytestmark = pytest.mark.gpu

L, D, N = 2047, 1 << 20, 16
EDGES = [0, 1, 15, 16, 17, 63, 64, 65535, 65536, 524287, 524288, 1048560, 1048575]
PER_CHANNEL = ("dx", "ddt", "dz", "dconv_w", "dconv_b", "ddt_bias", "dD", "dA")


def channels(seed):
    rng = np.random.default_rng(seed)
    extra = rng.choice(D, size=24 - len(EDGES), replace=False)
    return sorted(set(EDGES) | set(int(c) for c in extra))[:24]


def test_bwd_at_the_element_limit():
    need = 8 * L * D * 2 + L * D * 4 + 30 * (1 << 30)
    torch.cuda.empty_cache()  # blocks cached by earlier tests
    free, _ = torch.cuda.mem_get_info()
    if free < need:
        pytest.skip("needs %.1f GB of free device memory, %.1f GB free" % (need / 1e9, free / 1e9))
    print("bwd 1 x %d x %d d_state 16 bf16" % (L, D), flush=True)
    sys.stdout.flush()
    bf = torch.bfloat16
    seed = 3200
    lay = workloads.make_layer(1, 1, D, N, bf, seed=seed)
    g = torch.Generator(device="cuda").manual_seed(seed)
    io = dict(x=torch.randn(1, L, D, generator=g, device="cuda").to(bf),
              z=torch.randn(1, L, D, generator=g, device="cuda").to(bf),
              dt=(0.1 * torch.randn(1, L, D, generator=g, device="cuda")).to(bf),
              B=torch.randn(1, L, N, generator=g, device="cuda").to(bf),
              C=torch.randn(1, L, N, generator=g, device="cuda").to(bf))
    dy = torch.randn(1, L, D, generator=g, device="cuda").to(bf)
    prm = {k: lay[k].cuda() for k in H.PARAM_KEYS}
    got = ms.bwd(*(io[k] for k in H.IO_KEYS), ms.Params(*(prm[k] for k in H.PARAM_KEYS)), dy)
    torch.cuda.synchronize()
    ch = channels(seed)
    idx = torch.tensor(ch, device="cuda")
    sampled = {k: (got[k][..., idx].cpu() if k in ("dx", "ddt", "dz") else got[k][idx].cpu()) for k in PER_CHANNEL}
    dB, dC = got["dB"].cpu(), got["dC"].cpu()
    del got
    torch.cuda.empty_cache()

    # the checkpointing pair: the prefill (one unsplit chunk here) stores the
    # state every 16 steps and the backward reads them: equal bit for bit
    ck = ms.ckpt_like(io["x"])
    p_all = ms.Params(*(prm[k] for k in H.PARAM_KEYS))
    y_ck = ms.fwd(*(io[k] for k in H.IO_KEYS), p_all, ckpt=ck)[0]
    del y_ck
    got_ck = ms.bwd(*(io[k] for k in H.IO_KEYS), p_all, dy, ckpt=ck)
    torch.cuda.synchronize()
    for k in PER_CHANNEL:
        v = got_ck[k][..., idx] if k in ("dx", "ddt", "dz") else got_ck[k][idx]
        T.assert_bitwise(v.cpu(), sampled[k], "%s from checkpoints" % k)
    T.assert_bitwise(got_ck["dB"].cpu(), dB, "dB from checkpoints")
    T.assert_bitwise(got_ck["dC"].cpu(), dC, "dC from checkpoints")
    del got_ck, ck
    torch.cuda.empty_cache()

    # dB / dC: the two channel halves, each a call of its own
    halves = []
    for lo, hi in ((0, D // 2), (D // 2, D)):
        part = {k: (io[k][..., lo:hi].contiguous() if k in ("x", "dt", "z") else io[k]) for k in H.IO_KEYS}
        p = ms.Params(*(prm[k][lo:hi].contiguous() for k in H.PARAM_KEYS))
        r = ms.bwd(*(part[k] for k in H.IO_KEYS), p, dy[..., lo:hi].contiguous())
        torch.cuda.synchronize()
        halves.append((r["dB"].cpu(), r["dC"].cpu()))
        del part, p, r
        torch.cuda.empty_cache()
    T.assert_close(dB, halves[0][0].double() + halves[1][0].double(), 1e-3, "dB against the two halves")
    T.assert_close(dC, halves[0][1].double() + halves[1][1].double(), 1e-3, "dC against the two halves")

    # per-channel gradients against the oracle on the sampled channels
    sub = {k: (io[k][..., idx].cpu() if k in ("x", "dt", "z") else io[k].cpu()) for k in H.IO_KEYS}
    sub.update({k: lay[k][ch].contiguous() for k in H.PARAM_KEYS})
    dy_s = dy[..., idx].cpu()
    del io, dy
    torch.cuda.empty_cache()
    want = oracle.oracle_bwd(*(sub[k] for k in H.IO_KEYS + H.PARAM_KEYS), dy_s)
    for k in PER_CHANNEL:
        T.assert_close(sampled[k], want[k], T.RTOL[bf], "%s channels %s" % (k, ch))
