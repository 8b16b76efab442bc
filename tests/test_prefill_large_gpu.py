"""Prefill at the size limit: batch 1, seqlen 2047, d_inner 2^20, so
batch * seqlen * d_inner = 2,146,435,072, just under the 2^31 elements the ABI
accepts. One chunk of 2047 steps then spans 4 GiB (bfloat16) or 8 GiB (float32)
of every io tensor: the d_state 16 row kernel takes its per-stage-descriptor
path for real (not forced), and the d_state 8 quad kernel's per-stage
descriptors address rows far past 2^31 bytes. Outputs and final states of 24
channels (workgroup edges, both ends of d_inner, random ones) against the oracle.
The Mamba-2 SSD scan at its own limit (batch 4095 x seqlen 256 x 32 heads x 64)
on three batch rows, the last one at the far end of every tensor.

Inputs: parameters follow the shared recipe (workloads.make_layer, d_inner
2^20); x, z, B, C ~ N(0, 1) and dt ~ 0.1 N(0, 1) are drawn on the device from a
seeded generator and rounded to the io dtype; the sampled channels are gathered
on the device and copied to the host for the oracle.

Agreement rule: per element, |got - want| <= rtol * max(|want|, rms(want)),
rtol 1e-4 for float32 io and 2e-2 for bfloat16 io; the conv state bit for bit."""
import sys

import numpy as np
import pytest
import torch

import selective_state_space_07_amd as ms
import workloads
from tests import harness as H
from tests import tolerances as T

pytestmark = pytest.mark.gpu

L, D = 2047, 1 << 20
EDGES = [0, 1, 15, 16, 17, 63, 64, 65535, 65536, 524287, 524288, 1048560, 1048575]


def channels(seed):
    rng = np.random.default_rng(seed)
    extra = rng.choice(D, size=24 - len(EDGES), replace=False)
    return sorted(set(EDGES) | set(int(c) for c in extra))[:24]


@pytest.mark.parametrize("dtype,N", [(torch.bfloat16, 16), (torch.float32, 8)], ids=["bf16-n16-row", "f32-n8-quad"])
def test_prefill_at_the_element_limit(dtype, N):
    es = 2 if dtype == torch.bfloat16 else 4
    need = 4 * L * D * es + L * D * 4 + (2 << 30)
    torch.cuda.empty_cache()  # blocks cached by earlier tests
    free, _ = torch.cuda.mem_get_info()
    if free < need:
        pytest.skip("needs %.1f GB of free device memory, %.1f GB free" % (need / 1e9, free / 1e9))
    print("prefill 1 x %d x %d d_state %d %s" % (L, D, N, dtype), flush=True)
    sys.stdout.flush()
    seed = 3100 + N
    lay = workloads.make_layer(1, 1, D, N, dtype, seed=seed)
    g = torch.Generator(device="cuda").manual_seed(seed)
    io = dict(x=torch.randn(1, L, D, generator=g, device="cuda").to(dtype),
              z=torch.randn(1, L, D, generator=g, device="cuda").to(dtype),
              dt=(0.1 * torch.randn(1, L, D, generator=g, device="cuda")).to(dtype),
              B=torch.randn(1, L, N, generator=g, device="cuda").to(dtype),
              C=torch.randn(1, L, N, generator=g, device="cuda").to(dtype))
    p = ms.Params(*(lay[k].cuda() for k in H.PARAM_KEYS))
    y, cs, ss = ms.fwd(*(io[k] for k in H.IO_KEYS), p)
    torch.cuda.synchronize()
    ch = channels(seed)
    idx = torch.tensor(ch, device="cuda")
    sub = {k: (io[k][..., idx].cpu() if k in ("x", "dt", "z") else io[k].cpu()) for k in H.IO_KEYS}
    sub.update({k: lay[k][ch].contiguous() for k in H.PARAM_KEYS})
    y_s, cs_s, ss_s = y[..., idx].cpu(), cs[:, idx].cpu(), ss[:, idx].cpu()
    del io, y, cs, ss
    torch.cuda.empty_cache()
    yo, cso, sso = H.oracle_fwd(sub)
    rt = T.RTOL[dtype]
    T.assert_close(y_s, yo, rt, "y channels %s" % ch)
    T.assert_close(ss_s, sso, rt, "ssm_state channels %s" % ch)
    T.assert_bitwise(cs_s, cso, "conv_state channels %s" % ch)


@pytest.mark.parametrize("b,L,N,kind", [(70000, 1, 16, None), (70000, 2, 8, None), (66000, 3, 16, "lane")],
                         ids=["row-n16", "quad-n8", "lane-n16"])
def test_prefill_with_more_batch_rows_than_a_grid_extent_of_65535(b, L, N, kind):
    """The row, quad and lane kernels take the batch row from the grid's z
    extent: batch 66000-70000 (past the 65535 of a 16-bit extent), float32,
    every output element against the oracle and the conv state bit for bit."""
    print("prefill batch %d seqlen %d d_state %d kind %s" % (b, L, N, kind), flush=True)
    sys.stdout.flush()
    lay = workloads.make_layer(b, L, 16, N, torch.float32, seed=3400 + L)
    g = torch.Generator().manual_seed(3401)
    cs0, ss0 = torch.randn(b, 16, 3, generator=g), torch.randn(b, 16, N, generator=g)
    y, cs, ss = H.gpu_fwd(H.to_gpu(lay), cs0.cuda(), ss0.cuda(), testing_kind=kind)
    torch.cuda.synchronize()
    yo, cso, sso = H.oracle_fwd(lay, cs0, ss0)
    rt = T.RTOL[torch.float32]
    T.assert_close(y, yo, rt, "y batch %d" % b)
    T.assert_close(ss, sso, rt, "ssm_state batch %d" % b)
    T.assert_bitwise(cs, cso, "conv_state batch %d" % b)


SSD_B, SSD_L, SSD_H, SSD_N, SSD_G = 4095, 256, 32, 128, 2
SSD_ROWS = [0, 2047, 4094]


def test_ssd_at_the_element_limit():
    """Mamba-2 SSD scan with batch 4095, seqlen 256, 32 heads of 64, d_state
    128, two groups, bfloat16 io: batch * seqlen * nheads * headdim =
    2,146,959,360, just under 2^31. y and the final state of the first, a middle
    and the last batch row against the oracle on those rows."""
    need = 2 * SSD_B * SSD_L * SSD_H * 64 * 2 + SSD_B * SSD_L * SSD_H * 64 * 4 + 2 * SSD_B * SSD_H * 64 * SSD_N * 4
    torch.cuda.empty_cache()  # blocks cached by earlier tests
    free, _ = torch.cuda.mem_get_info()
    if free < need + (2 << 30):
        pytest.skip("needs %.1f GB of free device memory, %.1f GB free" % (need / 1e9, free / 1e9))
    print("ssd %d x %d x %d x 64 d_state %d bf16" % (SSD_B, SSD_L, SSD_H, SSD_N), flush=True)
    sys.stdout.flush()
    from oracle import ssd as ossd
    bf = torch.bfloat16
    lay = workloads.make_ssd(1, 1, SSD_H, 64, SSD_N, SSD_G, bf, seed=3300)
    g = torch.Generator(device="cuda").manual_seed(3300)
    io = dict(x=torch.randn(SSD_B, SSD_L, SSD_H, 64, generator=g, device="cuda").to(bf),
              dt=(0.1 * torch.randn(SSD_B, SSD_L, SSD_H, generator=g, device="cuda")).to(bf),
              B=torch.randn(SSD_B, SSD_L, SSD_G, SSD_N, generator=g, device="cuda").to(bf),
              C=torch.randn(SSD_B, SSD_L, SSD_G, SSD_N, generator=g, device="cuda").to(bf))
    y, s = ms.ssd_fwd(io["x"], io["dt"], io["B"], io["C"], *(lay[k].cuda() for k in ("dt_bias", "A", "D")))
    torch.cuda.synchronize()
    rows = torch.tensor(SSD_ROWS, device="cuda")
    sub = {k: v[rows].cpu() for k, v in io.items()}
    y_s, s_s = y[rows].cpu(), s[rows].cpu()
    del io, y, s
    torch.cuda.empty_cache()
    yo, so = ossd.oracle_ssd_fwd(sub["x"], sub["dt"], sub["B"], sub["C"], lay["dt_bias"], lay["A"], lay["D"])
    rt = T.RTOL[bf]
    T.assert_close(y_s, yo, rt, "ssd y rows %s" % SSD_ROWS)
    T.assert_close(s_s, so, rt, "ssd state rows %s" % SSD_ROWS)
