"""HIP path (through the C ABI) against the fp64 oracle on the same seeded
inputs: the five workloads at full size on every channel, their shapes again
with parameters drawn per channel, ragged shapes spanning several waves, chunks
and a ragged tail, both d_state values and both io dtypes. Apart from the five
workloads (which keep their own recipe), every case draws A[d, n], D and the
conv bias per channel."""
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


def check_fwd(layer_cpu, rtol, channels=None, with_states=False, seed=0, what="", **kw):
    layer = H.to_gpu(layer_cpu)
    cs = ss = None
    if with_states:
        g = torch.Generator().manual_seed(seed)
        bsz, d = layer_cpu["x"].shape[0], layer_cpu["x"].shape[2]
        n = layer_cpu["B"].shape[2]
        cs = torch.randn(bsz, d, 3, generator=g).cuda()
        ss = torch.randn(bsz, d, n, generator=g).cuda()
    y, cso, sso = H.gpu_fwd(layer, cs, ss, **kw)
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


def test_workload_long_full():
    """Workload 3 at full size (batch 1, L 65536, d 1536) in its timed launch
    configuration, every channel against the oracle."""
    cfg = workloads.WORKLOADS[3]
    say("workload 3", cfg["name"])
    s1, s2 = check_fwd(workloads.make_config(3), T.RTOL[cfg["dtype"]], what=cfg["name"])
    say("  y", s1, "\n  h", s2)


@pytest.mark.parametrize("index", [1, 2, 3])
def test_workload_shape_random_params(index):
    """The shapes of workloads 1-3 in their timed launch configurations with
    parameters drawn per channel (A[d, n] varies along d and n, D and the conv
    bias along d), every channel against the oracle: a kernel that indexed A
    by n alone or dropped or shared the D skip would fail here."""
    cfg = workloads.WORKLOADS[index]
    say("workload shape", index, cfg["name"], "random per-channel parameters")
    lay = workloads.make_layer(cfg["batch"], cfg["seqlen"], cfg["d_inner"], cfg["d_state"], cfg["dtype"],
                               seed=9100 + index, dt_range=cfg["dt_range"], params="random")
    s1, s2 = check_fwd(lay, T.RTOL[cfg["dtype"]], with_states=True, seed=index, what=cfg["name"] + " random")
    say("  y", s1, "\n  h", s2)


def test_workload_decode_full():
    """Workload 4 at full size: 24 layers of (GPU prefill of 128 tokens -> GPU
    step); the oracle runs prefill + step from its own states on every channel.
    The step kernel is also checked alone, fed the oracle's states."""
    cfg = workloads.WORKLOADS[4]
    rtol = T.RTOL[cfg["dtype"]]
    layers = workloads.make_decode_layers()
    for li, lay in enumerate(layers):
        say("decode layer", li)
        pre = H.to_gpu(dict(lay["prefill"], **lay["params"]))
        params = H.params_of(pre)
        _, cs, ss = H.gpu_fwd(pre)
        tok = H.to_gpu(lay["token"])
        y, cs2, ss2 = H.gpu_step(tok, params, cs, ss)
        torch.cuda.synchronize()
        # oracle: prefill then step from its own states
        _, cso, sso = H.oracle_fwd(pre)
        yo, cs2o, ss2o = H.oracle_step(lay["token"], lay["params"], torch.from_numpy(cso), torch.from_numpy(sso))
        T.assert_close(y, yo, rtol, "layer %d step y" % li)
        T.assert_close(ss2, ss2o, rtol, "layer %d step ssm_state" % li)
        T.assert_bitwise(cs2, cs2o, "layer %d step conv_state" % li)
        if li < 3:  # step alone from the oracle's (float32-rounded) states
            cs_in = torch.from_numpy(cso).float().cuda()
            ss_in = torch.from_numpy(sso).float().cuda()
            y1, c1, s1 = H.gpu_step(tok, params, cs_in, ss_in)
            torch.cuda.synchronize()
            yo1, co1, so1 = H.oracle_step(lay["token"], lay["params"], cs_in, ss_in)
            T.assert_close(y1, yo1, rtol, "layer %d step-alone y" % li)
            T.assert_close(s1, so1, rtol, "layer %d step-alone ssm_state" % li)
            T.assert_bitwise(c1, co1, "layer %d step-alone conv_state" % li)


XC_SHAPES = [
    # (batch, seqlen, d_inner, d_state, dtype): row kernel unsplit, quad kernel split, d_state 8
    (8, 300, 1536, 16, torch.bfloat16),
    (1, 1000, 100, 16, torch.float32),
    (3, 257, 70, 8, torch.bfloat16),
    (2, 5, 64, 16, torch.float32),
]


def strided_bc(B, C, width, off_b, off_c):
    """B and C [..., n] placed in the columns off_b and off_c of one device
    buffer [..., width] (the layout of x_proj's output); every other column
    holds NaN, so a read outside them shows in the outputs. Returns the buffer
    (kept alive by the caller) and the device addresses of B and C."""
    n = B.shape[-1]
    buf = torch.full(B.shape[:-1] + (width,), float("nan"), dtype=B.dtype)
    buf[..., off_b:off_b + n] = B
    buf[..., off_c:off_c + n] = C
    g = buf.cuda()
    es = g.element_size()
    return g, g.data_ptr() + off_b * es, g.data_ptr() + off_c * es


# (width, offset of B, offset of C) of the B / C rows; None = contiguous
BC_LAYOUTS = [None, (80, 48, 64), (37, 5, 21)]


@pytest.mark.parametrize("layout", BC_LAYOUTS, ids=["contiguous", "w80", "w37"])
@pytest.mark.parametrize("shape", XC_SHAPES, ids=[str(r[:4]) + str(r[4]).split(".")[-1] for r in XC_SHAPES])
def test_fwd_from_xc_matches_oracle(shape, layout):
    """mamba_scan_fwd_xc (the scan from a given activated conv output, as the
    mixer layer calls it) against oracle_fwd_xc on the same xc values, with an
    incoming SSM state; B and C contiguous or read in place from wider rows."""
    b, L, d, n, dtype = shape
    lay = workloads.make_layer(b, L, d, n, dtype, seed=L + d + 2, dt_range=(1e-4, 1e-1))
    g = torch.Generator().manual_seed(L)
    ss = torch.randn(b, d, n, generator=g)
    # any io values will do as xc: draw them like x
    xc = lay["x"]
    gl = H.to_gpu(lay)
    a = lambda t: t.data_ptr()
    if layout is None:
        stride, pB, pC = n, a(gl["B"]), a(gl["C"])
    else:
        width, ob, oc = layout
        if oc < ob + n:
            pytest.skip("B and C columns would overlap at d_state %d" % n)
        keep, pB, pC = strided_bc(lay["B"], lay["C"], width, ob, oc)
        stride = width
    y = torch.empty_like(gl["x"])
    sso = torch.empty(b, d, n, device="cuda")
    io = ms.MAMBA_BF16 if dtype == torch.bfloat16 else ms.MAMBA_F32
    need = ms.mamba_scan_fwd_workspace_bytes(b, L, d, n, io)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
    ssg = ss.cuda()
    ms.mamba_scan_fwd_xc(b, L, d, n, io, a(gl["x"]), a(gl["dt"]), a(gl["z"]), pB, pC, stride,
                         a(gl["dt_bias"]), a(gl["D"]), a(gl["A"]), a(ssg), a(y), a(sso), a(ws), need,
                         torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    import oracle
    yo, so = oracle.oracle_fwd_xc(xc, lay["dt"], lay["z"], lay["B"], lay["C"], lay["dt_bias"], lay["D"], lay["A"], ss)
    T.assert_close(y, yo, T.RTOL[dtype], "fwd_xc y %s %s" % (shape, layout))
    T.assert_close(sso, so, T.RTOL[dtype], "fwd_xc ssm_state %s %s" % (shape, layout))


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("n", [8, 16])
@pytest.mark.parametrize("inplace", [False, True])
@pytest.mark.parametrize("layout", BC_LAYOUTS, ids=["contiguous", "w80", "w37"])
def test_step_from_xc_matches_oracle(dtype, n, inplace, layout):
    """mamba_scan_step_xc (one token from its activated conv output) against
    oracle_fwd_xc over a sequence of length one, the SSM state updated into a
    new buffer or in place; B and C contiguous or read in place from wider
    rows (width 37: rows off the 4-element boundary, the scalar kernel)."""
    b, d = 5, 300
    lay = workloads.make_layer(b, 1, d, n, dtype, seed=70 + n)
    g = torch.Generator().manual_seed(n + 1)
    ss = torch.randn(b, d, n, generator=g)
    gl = H.to_gpu(lay)
    tok = {k: gl[k][:, 0].contiguous() for k in H.IO_KEYS}
    a = lambda t: t.data_ptr()
    if layout is None:
        stride, pB, pC = n, a(tok["B"]), a(tok["C"])
    else:
        width, ob, oc = layout
        if oc < ob + n:
            pytest.skip("B and C columns would overlap at d_state %d" % n)
        keep, pB, pC = strided_bc(lay["B"][:, 0], lay["C"][:, 0], width, ob, oc)
        stride = width
    y = torch.empty_like(tok["x"])
    ssg = ss.cuda()
    sso = ssg if inplace else torch.empty_like(ssg)
    io = ms.MAMBA_BF16 if dtype == torch.bfloat16 else ms.MAMBA_F32
    ms.mamba_scan_step_xc(b, d, n, io, a(tok["x"]), a(tok["dt"]), a(tok["z"]), pB, pC, stride,
                          a(gl["dt_bias"]), a(gl["D"]), a(gl["A"]), a(ssg), a(y), a(sso),
                          torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    import oracle
    yo, so = oracle.oracle_fwd_xc(lay["x"], lay["dt"], lay["z"], lay["B"], lay["C"], lay["dt_bias"], lay["D"],
                                  lay["A"], ss)
    T.assert_close(y, yo[:, 0], T.RTOL[dtype], "step_xc y %s" % (layout,))
    T.assert_close(sso, so, T.RTOL[dtype], "step_xc ssm_state %s" % (layout,))


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("n,rank", [(16, 48), (8, 7), (16, 1)])
@pytest.mark.parametrize("inplace", [False, True])
def test_step_with_dt_proj_matches_oracle(dtype, n, rank, inplace):
    """mamba_scan_step_xc_dtproj (dt = dt_low . w_dt[d] inside the step, rounded
    to the io dtype) against the oracle given that dt: dt_low, B and C read in
    place from one row per token (x_proj's output layout) and z from in_proj's
    (x, z) rows, the SSM state updated into a new buffer or in place; ranks 48
    (the measured layer's), 7 (not a multiple of the lanes sharing the dot
    product) and 1."""
    b, d = 6, 333
    width = rank + 2 * n
    g = torch.Generator().manual_seed(rank * 31 + n)
    lay = workloads.make_layer(b, 1, d, n, dtype, seed=90 + n + rank)
    dtl = (0.5 * torch.randn(b, rank, generator=g)).to(dtype)
    wdt = (torch.randn(d, rank, generator=g) / rank ** 0.5).to(dtype)
    row = torch.empty(b, width, dtype=dtype)
    row[:, :rank] = dtl
    row[:, rank:rank + n] = lay["B"][:, 0]
    row[:, rank + n:] = lay["C"][:, 0]
    ss = torch.randn(b, d, n, generator=g)
    gl = H.to_gpu(lay)
    tok = {k: gl[k][:, 0].contiguous() for k in ("x", "z")}
    rowg, wdtg = row.cuda(), wdt.cuda()
    es = rowg.element_size()
    y = torch.empty_like(tok["x"])
    ssg = ss.cuda()
    sso = ssg if inplace else torch.empty_like(ssg)
    io = ms.MAMBA_BF16 if dtype == torch.bfloat16 else ms.MAMBA_F32
    a = lambda t: t.data_ptr()
    # z read in place from rows (x, z) of 2 * d_inner, as a layer's in_proj writes them (NaN in the x half)
    xz = torch.full((b, 2 * d), float("nan"), dtype=dtype)
    xz[:, d:] = lay["z"][:, 0]
    xzg = xz.cuda()
    ms.mamba_scan_step_xc_dtproj(b, d, n, rank, io, a(tok["x"]), a(rowg), width, a(wdtg), a(xzg) + d * es, 2 * d,
                                 a(rowg) + rank * es, a(rowg) + (rank + n) * es, width, a(gl["dt_bias"]),
                                 a(gl["D"]), a(gl["A"]), a(ssg), a(y), a(sso), torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    import oracle
    # the oracle's dt: the float64 dot product, rounded to the io dtype where the layer would store it
    dt = (dtl.double() @ wdt.double().T).to(dtype)
    yo, so = oracle.oracle_fwd_xc(lay["x"], dt[:, None], lay["z"], lay["B"], lay["C"], lay["dt_bias"], lay["D"],
                                  lay["A"], ss)
    T.assert_close(y, yo[:, 0], T.RTOL[dtype], "step_xc_dtproj y")
    T.assert_close(sso, so, T.RTOL[dtype], "step_xc_dtproj ssm_state")


DTP_SHAPES = [
    # (batch, seqlen, d_inner, dtype, dt_rank): partial workgroups and ragged
    # last stages, ranks 8-64 (one or two 32-wide k blocks, a partly used
    # block), a split sequence (summary pass), the measured layer
    (2, 100, 40, torch.float32, 48),
    (2, 100, 40, torch.bfloat16, 48),
    (1, 300, 33, torch.bfloat16, 8),
    (3, 77, 20, torch.float32, 64),
    (2, 64, 16, torch.bfloat16, 40),
    (1, 2100, 48, torch.bfloat16, 48),
    (8, 2048, 1536, torch.bfloat16, 48),
]


@pytest.mark.parametrize("layout", ["row", "separate"])
@pytest.mark.parametrize("shape", DTP_SHAPES, ids=["-".join(map(str, s[:3])) + str(s[3]).split(".")[-1] + "-r%d" % s[4]
                                                   for s in DTP_SHAPES])
def test_fwd_with_dt_proj_matches_oracle(shape, layout):
    """mamba_scan_fwd_xc_dtproj (dt = dt_low . w_dt[d] on the matrix cores
    inside the prefill, rounded to the io dtype) against the oracle given that
    dt, with an incoming SSM state. "row": dt_low, B and C read in place from
    one row per token, with eight NaN columns right after dt_low (a read past
    dt_rank shows in the outputs), and z from rows (x, z) of 2 * d_inner with
    NaN in x; "separate": dt_low and z contiguous arrays of their own."""
    b, L, d, dtype, rank = shape
    n = 16
    lay = workloads.make_layer(b, L, d, n, dtype, seed=L + d + rank)
    g = torch.Generator().manual_seed(rank * 7 + L)
    dtl = (0.5 * torch.randn(b, L, rank, generator=g)).to(dtype)
    wdt = (torch.randn(d, rank, generator=g) / rank ** 0.5).to(dtype)
    ss = torch.randn(b, d, n, generator=g)
    gl = H.to_gpu(lay)
    a = lambda t: t.data_ptr()
    if layout == "row":
        width = rank + 8 + 2 * n
        row = torch.full((b, L, width), float("nan"), dtype=dtype)
        row[..., :rank] = dtl
        row[..., rank + 8:rank + 8 + n] = lay["B"]
        row[..., rank + 8 + n:] = lay["C"]
        rowg = row.cuda()
        es = rowg.element_size()
        p_dtl, dtl_stride = a(rowg), width
        pB, pC, bc_stride = a(rowg) + (rank + 8) * es, a(rowg) + (rank + 8 + n) * es, width
        # z in place from rows (x, z) of 2 * d_inner, NaN in the x half
        xz = torch.full((b, L, 2 * d), float("nan"), dtype=dtype)
        xz[..., d:] = lay["z"]
        xzg = xz.cuda()
        pz, z_stride = a(xzg) + d * es, 2 * d
    else:
        dtlg = dtl.cuda()
        p_dtl, dtl_stride = a(dtlg), rank
        pB, pC, bc_stride = a(gl["B"]), a(gl["C"]), n
        pz, z_stride = a(gl["z"]), d
    wdtg = wdt.cuda()
    y = torch.empty_like(gl["x"])
    sso = torch.empty(b, d, n, device="cuda")
    io = ms.MAMBA_BF16 if dtype == torch.bfloat16 else ms.MAMBA_F32
    need = ms.mamba_scan_fwd_workspace_bytes(b, L, d, n, io)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
    ssg = ss.cuda()
    print("fwd_xc_dtproj", shape, layout, flush=True)
    ms.mamba_scan_fwd_xc_dtproj(b, L, d, n, rank, io, a(gl["x"]), p_dtl, dtl_stride, a(wdtg), pz, z_stride, pB, pC,
                                bc_stride, a(gl["dt_bias"]), a(gl["D"]), a(gl["A"]), a(ssg), a(y), a(sso), a(ws), need,
                                torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    import oracle
    # the oracle's dt: the float64 dot product, rounded to the io dtype where a layer would store it
    dt = (dtl.double() @ wdt.double().T).to(dtype)
    yo, so = oracle.oracle_fwd_xc(lay["x"], dt, lay["z"], lay["B"], lay["C"], lay["dt_bias"], lay["D"], lay["A"], ss)
    T.assert_close(y, yo, T.RTOL[dtype], "fwd_xc_dtproj y %s %s" % (shape, layout))
    T.assert_close(sso, so, T.RTOL[dtype], "fwd_xc_dtproj ssm_state %s %s" % (shape, layout))


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_fwd_with_dt_proj_wide_rows_matches_oracle(dtype):
    """mamba_scan_fwd_xc_dtproj with rows far apart: z rows 2^24 elements
    apart (the largest stride accepted) make a 40-step chunk span more than
    2 GiB, so the kernel takes its per-stage buffer descriptors for z, dt_low
    and B/C (dt_low, B and C rows 2^20 elements apart); against the oracle,
    ragged (40 = 2 stages + 8 steps), with an incoming SSM state."""
    b, L, d, n, rank = 1, 40, 20, 16, 16
    zs, rs = 1 << 24, 1 << 20
    lay = workloads.make_layer(b, L, d, n, dtype, seed=404)
    g = torch.Generator().manual_seed(405)
    dtl = (0.5 * torch.randn(b, L, rank, generator=g)).to(dtype)
    wdt = (torch.randn(d, rank, generator=g) / rank ** 0.5).to(dtype)
    ss = torch.randn(b, d, n, generator=g)
    gl = H.to_gpu(lay)
    # exactly the extents the call may read: the last row ends d (z) or 3 * 16 (rows) elements in
    zbig = torch.zeros((b * L - 1) * zs + d, dtype=dtype, device="cuda")
    rows = torch.zeros((b * L - 1) * rs + rank + 2 * n, dtype=dtype, device="cuda")
    for t in range(L):
        zbig[t * zs:t * zs + d] = gl["z"][0, t]
        rows[t * rs:t * rs + rank] = dtl[0, t].cuda()
        rows[t * rs + rank:t * rs + rank + n] = gl["B"][0, t]
        rows[t * rs + rank + n:t * rs + rank + 2 * n] = gl["C"][0, t]
    es = rows.element_size()
    a = lambda t: t.data_ptr()
    wdtg = wdt.cuda()
    y = torch.empty_like(gl["x"])
    sso = torch.empty(b, d, n, device="cuda")
    io = ms.MAMBA_BF16 if dtype == torch.bfloat16 else ms.MAMBA_F32
    need = ms.mamba_scan_fwd_workspace_bytes(b, L, d, n, io)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
    ssg = ss.cuda()
    print("fwd_xc_dtproj wide rows", dtype, flush=True)
    ms.mamba_scan_fwd_xc_dtproj(b, L, d, n, rank, io, a(gl["x"]), a(rows), rs, a(wdtg), a(zbig), zs,
                                a(rows) + rank * es, a(rows) + (rank + n) * es, rs, a(gl["dt_bias"]), a(gl["D"]),
                                a(gl["A"]), a(ssg), a(y), a(sso), a(ws), need, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    del zbig, rows
    import oracle
    dt = (dtl.double() @ wdt.double().T).to(dtype)
    yo, so = oracle.oracle_fwd_xc(lay["x"], dt, lay["z"], lay["B"], lay["C"], lay["dt_bias"], lay["D"], lay["A"], ss)
    T.assert_close(y, yo, T.RTOL[dtype], "fwd_xc_dtproj wide y")
    T.assert_close(sso, so, T.RTOL[dtype], "fwd_xc_dtproj wide ssm_state")


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
    lay = workloads.make_layer(b, L, d, n, dtype, seed=b * 1009 + L * 17 + d * 3 + n, dt_range=(1e-4, 1e-1))
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
def test_forced_kernel_family(kind, shape):
    """Every prefill kernel family, chosen through the testing entry point, on
    shapes that the default plan sends elsewhere (so each family's split and
    unsplit paths run), with incoming states."""
    b, L, d, n, dtype = shape
    if kind == "row" and n != 16:
        pytest.skip("the row kernel serves d_state 16 only")
    say("forced", kind, shape, "workspace", ms.workspace_bytes(b, L, d, n, dtype, testing_kind=kind))
    lay = workloads.make_layer(b, L, d, n, dtype, seed=L + d, dt_range=(1e-4, 1e-1))
    check_fwd(lay, T.RTOL[dtype], with_states=True, seed=L, what="%s %s" % (kind, shape), testing_kind=kind)


@pytest.mark.parametrize("shape", [(8, 300, 1536, 16, torch.bfloat16), (2, 300, 96, 16, torch.float32)])
def test_row_wide_path_bitwise(shape):
    """The row kernel's per-stage-descriptor path (taken when a chunk spans
    2 GiB or more) gives bit-identical results to the chunk-wide one."""
    b, L, d, n, dtype = shape
    lay = H.to_gpu(workloads.make_layer(b, L, d, n, dtype, seed=5, dt_range=(1e-4, 1e-1)))
    g = torch.Generator().manual_seed(1)
    cs = torch.randn(b, d, 3, generator=g).cuda()
    ss = torch.randn(b, d, n, generator=g).cuda()
    y1, c1, s1 = H.gpu_fwd(lay, cs, ss, testing_kind="row")
    y2, c2, s2 = H.gpu_fwd(lay, cs, ss, testing_kind="row", testing_force_wide=True)
    torch.cuda.synchronize()
    T.assert_bitwise(y2, y1, "wide y")
    T.assert_bitwise(s2, s1, "wide ssm_state")
    T.assert_bitwise(c2, c1, "wide conv_state")
