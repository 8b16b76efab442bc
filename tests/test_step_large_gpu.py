"""Decode steps whose lane index passes 2^31, each with about 34.6 GB of
float32 state updated in place, bfloat16 io:

- Mamba-1, 66000 x 8192 channels, d_state 16: four lanes per channel, so the
  index passes 2^31 from channel 2^29 on (batch row 65536);
- Mamba-2 SSD, batch 44000, 24 heads of 64, d_state 128: 32 lanes per state
  row, past 2^31 from row 2^26 on (inside batch row 43690).

Both launches also spread their workgroups over two grid dimensions (2^22 along
x; the first split falls in batch row 32768, respectively 21845). The batch rows
holding those points, and the first and last rows, are checked against the
oracle.

Inputs: parameters follow the shared recipes (workloads.make_layer with d_inner
8192, workloads.make_ssd with 24 heads); the token (x, z, B, C ~ N(0, 1),
dt ~ 0.1 N(0, 1), rounded to bfloat16) and the states (~ N(0, 1), float32) are
drawn on the device from a seeded generator, and the sampled rows are copied to
the host before the in-place update.

Agreement rule: per element, |got - want| <= 2e-2 * max(|want|, rms(want)) for
y and the ssm state; the conv state bit for bit."""
import sys

import pytest
import torch

import selective_state_space_07_amd as ms
import workloads
from oracle import ssd as ossd
from tests import harness as H
from tests import tolerances as T

pytestmark = pytest.mark.gpu

BATCH, D_INNER, D_STATE = 66000, 8192, 16
ROWS = [0, 32768, 65535, 65536, 65999]


def need_free(nbytes):
    torch.cuda.empty_cache()  # blocks cached by earlier tests
    free, _ = torch.cuda.mem_get_info()
    if free < nbytes:
        pytest.skip("needs %.1f GB of free device memory, %.1f GB free" % (nbytes / 1e9, free / 1e9))


def test_step_past_2_31_lanes():
    need_free(BATCH * D_INNER * (D_STATE + 3) * 4 + 4 * BATCH * D_INNER * 2 + (1 << 30))
    print("step 66000 x 8192 x 16 bf16 in place", flush=True)
    sys.stdout.flush()
    lay = workloads.make_layer(1, 1, D_INNER, D_STATE, torch.bfloat16, seed=2931)
    params_cpu = {k: lay[k] for k in H.PARAM_KEYS}
    p = ms.Params(*(lay[k].cuda() for k in ("conv_w", "conv_b", "dt_bias", "D", "A")))
    g = torch.Generator(device="cuda").manual_seed(2931)
    bf = torch.bfloat16
    tok = dict(x=torch.randn(BATCH, D_INNER, generator=g, device="cuda").to(bf),
               z=torch.randn(BATCH, D_INNER, generator=g, device="cuda").to(bf),
               dt=(0.1 * torch.randn(BATCH, D_INNER, generator=g, device="cuda")).to(bf),
               B=torch.randn(BATCH, D_STATE, generator=g, device="cuda").to(bf),
               C=torch.randn(BATCH, D_STATE, generator=g, device="cuda").to(bf))
    cs = torch.randn(BATCH, D_INNER, 3, generator=g, device="cuda")
    ss = torch.randn(BATCH, D_INNER, D_STATE, generator=g, device="cuda")
    rows = torch.tensor(ROWS, device="cuda")
    tok_cpu = {k: v[rows].cpu() for k, v in tok.items()}
    cs_cpu, ss_cpu = cs[rows].cpu(), ss[rows].cpu()
    y, cs2, ss2 = ms.step(tok["x"], tok["dt"], tok["z"], tok["B"], tok["C"], p, cs, ss, inplace=True)
    torch.cuda.synchronize()
    assert cs2 is cs and ss2 is ss
    y_s, cs_s, ss_s = y[rows].cpu(), cs[rows].cpu(), ss[rows].cpu()
    del tok, cs, ss, cs2, ss2, y
    torch.cuda.empty_cache()
    yo, cso, sso = H.oracle_step(tok_cpu, params_cpu, cs_cpu, ss_cpu)
    rt = T.RTOL[torch.bfloat16]
    T.assert_close(y_s, yo, rt, "y rows %s" % ROWS)
    T.assert_close(ss_s, sso, rt, "ssm_state rows %s" % ROWS)
    T.assert_bitwise(cs_s, cso, "conv_state rows %s" % ROWS)


SSD_BATCH, SSD_HEADS, SSD_N = 44000, 24, 128
SSD_ROWS = [0, 21845, 43690, 43999]


def test_ssd_step_past_2_31_lanes():
    need_free(SSD_BATCH * SSD_HEADS * 64 * SSD_N * 4 + (1 << 30))
    print("ssd step 44000 x 24 x 64 x 128 bf16 in place", flush=True)
    sys.stdout.flush()
    lay = workloads.make_ssd(1, 1, SSD_HEADS, 64, SSD_N, 1, torch.bfloat16, seed=2932)
    prm = {k: lay[k] for k in ("dt_bias", "A", "D")}
    g = torch.Generator(device="cuda").manual_seed(2932)
    bf = torch.bfloat16
    tok = dict(x=torch.randn(SSD_BATCH, SSD_HEADS, 64, generator=g, device="cuda").to(bf),
               dt=(0.1 * torch.randn(SSD_BATCH, SSD_HEADS, generator=g, device="cuda")).to(bf),
               B=torch.randn(SSD_BATCH, 1, SSD_N, generator=g, device="cuda").to(bf),
               C=torch.randn(SSD_BATCH, 1, SSD_N, generator=g, device="cuda").to(bf))
    st = torch.randn(SSD_BATCH, SSD_HEADS, 64, SSD_N, generator=g, device="cuda")
    rows = torch.tensor(SSD_ROWS, device="cuda")
    tok_cpu = {k: v[rows].cpu() for k, v in tok.items()}
    st_cpu = st[rows].cpu()
    y, st2 = ms.ssd_step(tok["x"], tok["dt"], tok["B"], tok["C"], *(prm[k].cuda() for k in ("dt_bias", "A", "D")),
                         st, inplace=True)
    torch.cuda.synchronize()
    assert st2 is st
    y_s, st_s = y[rows].cpu(), st[rows].cpu()
    del tok, st, st2, y
    torch.cuda.empty_cache()
    yo, so = ossd.oracle_ssd_step(tok_cpu["x"], tok_cpu["dt"], tok_cpu["B"], tok_cpu["C"], prm["dt_bias"], prm["A"],
                                  prm["D"], st_cpu)
    rt = T.RTOL[torch.bfloat16]
    T.assert_close(y_s, yo, rt, "ssd y rows %s" % SSD_ROWS)
    T.assert_close(st_s, so, rt, "ssd state rows %s" % SSD_ROWS)
