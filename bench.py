"""Throughput of the selective-scan mixer core on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--workloads 1,0,2,3,4] [--no-cpu-baseline]

A step is one prefill call (conv + SiLU, softplus, the selective scan with its
readout and D skip, the gate, and the final states) over one batch of the
130M-class workload (batch 8, seqlen 2048, d_inner 1536, d_state 16, bf16 io,
float32 state), with inputs resident in HBM. K steps are timed with HIP events
on the stream the library launches on; the inputs rotate over several copies
whose total size exceeds the 256 MB last-level cache, so every step reads
from HBM. Prints ONE JSON line. The other workloads are reported inside it
under "workloads" (the decode workload as one 24-layer step).
"""
import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 matrix peak (no sparsity)
# fp32 vector peak: 157.3 TFLOP/s = 256 CUs x 4 SIMDs x 32 lane-FMAs x 2.4 GHz. On gfx950 plain
# (unpacked) fp32 instructions whose operands are all VGPRs reach that rate from two or more waves
# per SIMD (bench.py --valu-probe); a slot is one lane-operation at that rate.
PEAK_VALU_GSLOTS = 256 * 4 * 32 * 2.4
# exp2 / log2 / rcp issue at a quarter of that rate (same probe): 4 slots each
TRANS_SLOTS = 4
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.json")
CALIB_TAG = "AbsFunctor"  # the calibration kernel: torch's elementwise |x|


# The sources of the kernel whose HBM traffic profiles/hbm_traffic.json records
# for each workload (the prefill plan and the row kernel; the decode step).
TRAFFIC_SOURCES = {1: ("scan_device.h", "scan_fwd_common.h", "scan_fwd.hip", "scan_fwd_row.hip"),
                   4: ("scan_device.h", "scan_step.hip")}


def kernel_digest(idx):
    """sha256 over the sources of workload idx's recorded kernel: HBM counters
    taken on other sources no longer apply."""
    import hashlib
    d = os.path.join(ROOT, "selective_state_space_07_amd", "csrc")
    h = hashlib.sha256()
    for f in TRAFFIC_SOURCES[idx]:
        h.update(f.encode())
        with open(os.path.join(d, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def pmc_summary(fetch_csv, write_csv, calib_bytes):
    """Average FETCH_SIZE / WRITE_SIZE (KiB per dispatch) of every kernel in two
    rocprofv3 counter-collection CSVs, each scaled by calib_bytes / (what the
    same counter reads for the calibration copy)."""
    import csv
    out = {}
    for counter, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        per = {}
        with open(path) as fh:
            for r in csv.DictReader(fh):
                if r["Counter_Name"] == counter:
                    per.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]) * 1024.0)
        calib = [v for k, vs in per.items() if CALIB_TAG in k for v in vs]
        if not calib:
            raise SystemExit("no calibration dispatch in %s" % path)
        factor = calib_bytes / (sum(calib) / len(calib))
        out[counter] = dict(calibration_factor=factor, calibration_dispatches=len(calib), kernels={
            k: dict(dispatches=len(vs), raw_bytes_avg=sum(vs) / len(vs), bytes_avg=factor * sum(vs) / len(vs),
                    raw_bytes_min=min(vs), raw_bytes_max=max(vs))
            for k, vs in per.items() if "mscan" in k})
    return out


def traffic_alg_bytes(idx):
    """(workload name, algorithmic read bytes, algorithmic write bytes) of one
    launch of workload idx's dominant kernel (idx 4: one layer's decode step)."""
    import workloads
    cfg = workloads.WORKLOADS[idx]
    b, d, n = cfg["batch"], cfg["d_inner"], cfg["d_state"]
    io = 2 if "bf16" in cfg["name"] else 4
    if idx == 4:
        alg = decode_bytes_per_layer(b, d, n, io)
        write = b * d * (3 + n) * 4 + b * d * io
    else:
        L = cfg["seqlen"]
        alg = algorithmic_bytes(b, L, d, n, io)
        write = b * L * d * io + b * d * (3 + n) * 4
    return cfg["name"], alg - write, write


TRAFFIC_KERNEL = {1: "scan_row_kernel", 4: "scan_step_vec_kernel"}


def update_traffic(idx, counters, calib_bytes, kernel_stats=None):
    """Record, in profiles/hbm_traffic.json, the HBM bytes per dispatch of
    workload idx's dominant kernel (the decode workload's priming prefills
    are not it)."""
    fetch, write = counters["FETCH_SIZE"], counters["WRITE_SIZE"]
    tag = TRAFFIC_KERNEL[idx]
    kname = max((k for k in fetch["kernels"] if tag in k),
                key=lambda k: fetch["kernels"][k]["raw_bytes_avg"] * fetch["kernels"][k]["dispatches"])
    fk, wk = fetch["kernels"][kname], write["kernels"][kname]
    name, alg_r, alg_w = traffic_alg_bytes(idx)
    entry = dict(kernel=kname, fetch_bytes=fk["bytes_avg"], write_bytes=wk["bytes_avg"],
                 fetch_raw_bytes=fk["raw_bytes_avg"], write_raw_bytes=wk["raw_bytes_avg"],
                 fetch_factor=fetch["calibration_factor"], write_factor=write["calibration_factor"],
                 alg_read_bytes=alg_r, alg_write_bytes=alg_w, dispatches=fk["dispatches"],
                 sources_sha256=kernel_digest(idx))
    if kernel_stats:
        import csv
        with open(kernel_stats) as fh:
            for r in csv.DictReader(fh):
                if r["Name"] == kname:
                    entry["avg_duration_ns"] = float(r["AverageNs"])
    t = dict(calibration_copy_bytes=calib_bytes, workloads={})
    if os.path.exists(TRAFFIC_FILE):
        with open(TRAFFIC_FILE) as fh:
            old = json.load(fh)
        t["workloads"] = {k: v for k, v in old.get("workloads", {}).items() if "sources_sha256" in v}
    t["workloads"][name] = entry
    with open(TRAFFIC_FILE, "w") as fh:
        json.dump(t, fh, indent=1)
        fh.write("\n")
    return entry


def sq_summary(path, idx):
    """Average of every counter per dispatch of each library kernel in a
    rocprofv3 counter-collection CSV; for workload idx's prefill, also per
    wave and per 16-step stage (the row and quad kernels' unit of work)."""
    import csv
    import workloads
    per = {}
    for r in csv.DictReader(open(path)):
        if "mscan" not in r["Kernel_Name"]:
            continue
        k = per.setdefault(r["Kernel_Name"], {})
        k.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    cfg = workloads.WORKLOADS[idx]
    out = {}
    for kname, cs in per.items():
        avg = {c: sum(v) / len(v) for c, v in cs.items()}
        e = dict(dispatches=max(len(v) for v in cs.values()), per_dispatch=avg)
        waves = avg.get("SQ_WAVES")
        if waves and idx != 4:
            stages = -(-cfg["seqlen"] // 16)
            e["per_wave_stage"] = {c: v / waves / stages for c, v in avg.items() if c != "SQ_WAVES"}
        out[kname] = e
    return dict(workload=cfg["name"], kernels=out)


def traffic_entry(idx):
    """Measured HBM bytes per dispatch of workload idx's dominant kernel, if
    they were taken on its current sources; else None."""
    if idx not in TRAFFIC_SOURCES or not os.path.exists(TRAFFIC_FILE):
        return None
    import workloads
    with open(TRAFFIC_FILE) as fh:
        t = json.load(fh)
    e = t.get("workloads", {}).get(workloads.WORKLOADS[idx]["name"])
    if e is None or e.get("sources_sha256") != kernel_digest(idx):
        return None
    return e


def algorithmic_bytes(batch, seqlen, d_inner, d_state, io_bytes):
    """Bytes the method must move once: x, dt, z read and y written (io dtype),
    B and C (io dtype), the float32 parameters, and the float32 final states."""
    bld = batch * seqlen * d_inner
    return (4 * bld * io_bytes + 2 * batch * seqlen * d_state * io_bytes
            + d_inner * (4 + 3) * 4 + d_inner * d_state * 4 + batch * d_inner * (3 + d_state) * 4)


def decode_bytes_per_layer(batch, d_inner, d_state, io_bytes):
    """One token: states read and written (float32), x/dt/z read and y written,
    B/C rows, parameters."""
    bd = batch * d_inner
    return (2 * bd * (3 + d_state) * 4 + 4 * bd * io_bytes + 2 * batch * d_state * io_bytes
            + d_inner * (4 + 3) * 4 + d_inner * d_state * 4)


def algorithmic_ops(d_state):
    """Minimal fp32 VALU operations per element of the prefill, as (plain,
    transcendental): conv 4 FMA; SiLU(u) = u / (1 + exp(-u)) 3 + exp, rcp;
    softplus in its stable form 6 + exp, log; delta*xc 1; per state n:
    delta*A, (delta*xc)*B, the state FMA and the readout FMA 4 + exp; D skip 1;
    SiLU(z) 3 + exp, rcp; gate 1."""
    plain = 4 + 3 + 6 + 1 + 4 * d_state + 1 + 3 + 1
    trans = 2 + 2 + d_state + 2
    return plain, trans


def algorithmic_slots(d_state):
    """Minimal VALU slots per element of the prefill (plain op 1 slot,
    transcendental TRANS_SLOTS): 171 at d_state 16."""
    plain, trans = algorithmic_ops(d_state)
    return plain + TRANS_SLOTS * trans


def algorithmic_slots_bwd(d_state):
    """Minimal VALU slots per element of the backward (same pricing): the
    forward recomputed (algorithmic_slots) plus, per state n, the adjoint
    dh += C dy' (1), the dC term h dy' (1), the decay term dh a h_prev (2)
    with its sum over n (1), dA += delta * that (1), the input term dh B (1)
    with its sum over n (1), the dB term dh delta xc (1) and dh *= a (1) = 10
    plain; per element: dz (gate derivative, SiLU(z) reused) 6, dD 1, dxc 2,
    ddelta 2, softplus derivative (a sigmoid: 4 plain and a reciprocal), SiLU
    derivative 5, the four conv taps' weight and input gradients 8, dconv_b
    and ddt_bias 2 = 30 plain and 1 transcendental."""
    return algorithmic_slots(d_state) + 10 * d_state + 30 + TRANS_SLOTS


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--warm-seconds", type=float, default=WARM_SECONDS,
                    help="every warm-up also lasts at least this many seconds of device work (the shader clock "
                         "ramps up over the first ~40 ms of sustained load); 0 = exactly --warmup calls")
    ap.add_argument("--workloads", default="1,0,2,3,4,1p,m1,m4,b1,s1,s4",
                    help="first one is the headline; a trailing p = the same prefill over packed documents; "
                         "m1 / m4 = a whole 130M-class mixer layer, prefill / decode; b1 = the backward of "
                         "the 130M-class prefill; s1 / s4 = the Mamba-2 SSD scan, prefill / decode step")
    ap.add_argument("--rotate-bytes", type=float, default=1.0e9, help="total bytes of rotated input copies")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--only", default=None,
                    help="profile mode: run just this workload for --steps calls and print its timing")
    ap.add_argument("--copy-calib", type=float, default=0.0,
                    help="profile mode: also run a plain elementwise copy (|x| of a float32 buffer) of this many "
                         "bytes read and written, as the HBM counter calibration")
    ap.add_argument("--valu-probe", action="store_true",
                    help="measure the fp32 VALU issue rate (FMA, exp2, log2, rcp; 1-8 waves per SIMD) and the "
                         "shader clock with libmamba_probe.so; prints one JSON line")
    ap.add_argument("--update-traffic", action="store_true",
                    help="with --pmc-summary and --only W (1 or 4): record the bytes of W's dominant kernel in "
                         "profiles/hbm_traffic.json")
    ap.add_argument("--kernel-stats", default=None,
                    help="with --update-traffic: the rocprofv3 kernel_stats.csv of W, whose average duration of "
                         "that kernel is recorded beside its bytes")
    ap.add_argument("--sq-summary", default=None, metavar="CSV",
                    help="summarise a rocprofv3 --pmc counter-collection CSV of --only W: each counter's average "
                         "per dispatch of each library kernel, and per wave and 16-step stage for the prefill "
                         "kernels of workload W; prints one JSON line")
    ap.add_argument("--pmc-summary", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="summarise two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) of --only W --copy-calib "
                         "BYTES into HBM bytes per dispatch of each library kernel; prints one JSON line")
    return ap.parse_args()


# Minimum length of every warm-up, in seconds of device work (--warm-seconds).
# The shader clock of an MI355X under sustained load ramps up over the first
# ~40 ms: a workload timed from a cold start runs 10-20% slower for that long.
WARM_SECONDS = 0.1


def warm_up(run, warmup):
    """At least `warmup` calls of run(i), and more until WARM_SECONDS of
    device time have passed after the first batch (which may carry one-off
    library and module set-up); calls in batches of 8, each waited for."""
    import torch
    i = 0
    t0 = None
    while i < warmup or t0 is None or time.perf_counter() - t0 < WARM_SECONDS:
        for _ in range(8):
            run(i)
            i += 1
        torch.cuda.synchronize()
        if t0 is None:
            t0 = time.perf_counter()
    return i


def timed(run, steps, warmup, stream):
    """Average ms per call of run(i) over `steps` calls, HIP events on `stream`,
    after the warm-up (warm_up)."""
    import torch
    warm_up(run, warmup)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(steps):
        run(i)
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def launch_timed(run, steps, warmup, stream):
    """Average ms of one call's device work: each call bracketed by its own
    pair of HIP events on `stream`, so the gaps between calls (host cost,
    dispatch) are left out. For a one-kernel call this is the kernel's launch
    duration, the figure a rocprofv3 kernel trace averages."""
    import torch
    warm_up(run, warmup)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for i in range(steps):
        ev[i][0].record(stream)
        run(i)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    return sum(a.elapsed_time(b) for a, b in ev) / steps


def graph_timed(run, calls, steps, warmup, stream):
    """Average ms per call of run(0..calls-1) captured once in a HIP graph and
    replayed `steps` times: the device time of the launches without the host
    cost of the Python wrapper and the ctypes call (which a small launch does
    not hide)."""
    import torch
    for i in range(calls):
        run(i)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(calls):
            run(i)
    torch.cuda.synchronize()
    return timed(lambda i: g.replay(), steps, warmup, stream) / calls


def copy_rate(launch_bytes, launches, steps, warmup, stream):
    """GB/s of a plain device copy moving `launch_bytes` per launch (half read,
    half written), `launches` launches per step on distinct buffers: what
    launches of that size reach at all, beside the kernel's own rate."""
    import torch
    per = launch_bytes // 8  # float32 elements read (and written) per launch
    bufs = [(torch.ones(per, device="cuda"), torch.empty(per, device="cuda")) for _ in range(launches)]

    def run(i):
        for src, dst in bufs:
            (dst.copy_(src) if i % 2 == 0 else src.copy_(dst))

    t = timed(run, steps, warmup, stream) * 1e-3
    return launches * per * 8 / t / 1e9


def bench_prefill(index, steps, warmup, rotate_bytes, packed=False):
    """One prefill call per step; with `packed`, over packed documents
    (mamba_scan_fwd_seq, per-row document boundaries at different places)."""
    import torch
    import selective_state_space_07_amd as ms
    import workloads
    cfg = workloads.WORKLOADS[index]
    b, L, d, n, dtype = cfg["batch"], cfg["seqlen"], cfg["d_inner"], cfg["d_state"], cfg["dtype"]
    io_bytes = 2 if dtype == torch.bfloat16 else 4
    alg = algorithmic_bytes(b, L, d, n, io_bytes)
    lay = workloads.make_config(index)
    copies = max(1, min(8, math.ceil(rotate_bytes / alg)))
    sets = []
    for c in range(copies):
        g = {k: v.cuda() for k, v in lay.items()}
        y = torch.empty_like(g["x"])
        cso = torch.empty(b, d, 3, device="cuda")
        sso = torch.empty(b, d, n, device="cuda")
        sets.append((g, y, cso, sso))
    params = ms.Params(*(sets[0][0][k] for k in ("conv_w", "conv_b", "dt_bias", "D", "A")))
    seq = None
    if packed:
        seq = torch.from_numpy(workloads.make_seq_idx("misaligned_rows", b, L, seed=11)).cuda()
    ws = torch.empty(max(1, ms.workspace_bytes(b, L, d, n, dtype)), device="cuda", dtype=torch.uint8)
    stream = torch.cuda.current_stream()

    def run(i):
        g, y, cso, sso = sets[i % copies]
        ms.fwd(g["x"], g["dt"], g["z"], g["B"], g["C"], params, out=y, conv_state_out=cso, ssm_state_out=sso,
               workspace=ws, seq_idx=seq)

    ms_step = timed(run, steps, warmup, stream)
    launch_ms = launch_timed(run, steps, warmup, stream)
    graph_ms = graph_timed(run, copies, steps, warmup, stream)
    elems = b * L * d
    t = ms_step * 1e-3
    tg = graph_ms * 1e-3
    tk = launch_ms * 1e-3
    slots = algorithmic_slots(n) * elems
    return dict(workload=cfg["name"] + ("_packed_docs" if packed else ""), batch=b, seqlen=L, d_inner=d, d_state=n,
                io_dtype="bf16" if io_bytes == 2 else "f32", ms_per_step=ms_step, elems_per_s=elems / t,
                alg_bytes=alg, hbm_gbs=alg / t / 1e9, hbm_frac=alg / t / 1e9 / PEAK_HBM_GBS,
                alg_valu_slots=slots, valu_gslots=slots / t / 1e9, valu_frac=slots / t / 1e9 / PEAK_VALU_GSLOTS,
                input_copies=copies,
                launch_ms=launch_ms, launch_hbm_gbs=alg / tk / 1e9, launch_hbm_frac=alg / tk / 1e9 / PEAK_HBM_GBS,
                launch_valu_gslots=slots / tk / 1e9, launch_valu_frac=slots / tk / 1e9 / PEAK_VALU_GSLOTS,
                graph_ms_per_call=graph_ms, graph_elems_per_s=elems / tg, graph_hbm_frac=alg / tg / 1e9 / PEAK_HBM_GBS,
                graph_valu_frac=slots / tg / 1e9 / PEAK_VALU_GSLOTS)


def bench_decode(steps, warmup):
    import torch
    import selective_state_space_07_amd as ms
    import workloads
    cfg = workloads.WORKLOADS[4]
    layers = workloads.make_decode_layers()
    b, d, n = cfg["batch"], cfg["d_inner"], cfg["d_state"]
    state = []
    for lay in layers:
        pre = {k: v.cuda() for k, v in lay["prefill"].items()}
        p = ms.Params(*(lay["params"][k].cuda() for k in ("conv_w", "conv_b", "dt_bias", "D", "A")))
        _, cs, ss = ms.fwd(pre["x"], pre["dt"], pre["z"], pre["B"], pre["C"], p)
        tok = {k: v.cuda() for k, v in lay["token"].items()}
        y = torch.empty_like(tok["x"])
        state.append((tok, p, cs, ss, torch.empty_like(cs), torch.empty_like(ss), y))
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()

    def run(i):
        # one 24-layer decode step; states ping-pong between two buffers
        for li, (tok, p, cs, ss, cs2, ss2, y) in enumerate(state):
            src, dst = ((cs, ss), (cs2, ss2)) if i % 2 == 0 else ((cs2, ss2), (cs, ss))
            ms.mamba_scan_step(b, d, n, 4, ms.MAMBA_BF16, tok["x"].data_ptr(), tok["dt"].data_ptr(),
                               tok["z"].data_ptr(), tok["B"].data_ptr(), tok["C"].data_ptr(), p.conv_w.data_ptr(),
                               p.conv_b.data_ptr(), p.dt_bias.data_ptr(), p.D.data_ptr(), p.A.data_ptr(),
                               src[0].data_ptr(), src[1].data_ptr(), y.data_ptr(), dst[0].data_ptr(),
                               dst[1].data_ptr(), stream.cuda_stream)

    ms_step = timed(run, steps, warmup, stream)
    t = ms_step * 1e-3
    alg = len(layers) * decode_bytes_per_layer(b, d, n, 2)
    elems = len(layers) * b * d
    copy_gbs = copy_rate(decode_bytes_per_layer(b, d, n, 2), len(layers), steps, warmup, stream)
    return dict(workload=cfg["name"], layers=len(layers), batch=b, d_inner=d, d_state=n, io_dtype="bf16",
                ms_per_step=ms_step, elems_per_s=elems / t, alg_bytes=alg, hbm_gbs=alg / t / 1e9,
                hbm_frac=alg / t / 1e9 / PEAK_HBM_GBS, copy_same_size_gbs=copy_gbs,
                frac_of_copy=alg / t / 1e9 / copy_gbs)


def bench_mixer(kind, steps, warmup):
    """A whole 130M-class mixer layer (d_model 768, d_inner 1536, d_state 16,
    dt_rank 48, bf16): kind "m1" = prefill of batch 8 x 2048 tokens, "m4" = one
    decode token for batch 256 (states ping-pong). Times the layer (five rocBLAS
    GEMMs, the conv kernel, the scan) and reports the GEMM flop rate."""
    import torch
    import workloads
    from selective_state_space_07_amd import mixer
    dm, d, n, r = 768, 1536, 16, 48
    b, L = (8, 2048) if kind == "m1" else (256, 1)
    lay = workloads.make_mixer_layer(b, L, dm, d, n, r, torch.bfloat16, seed=17, conv_bias=0.1, params="config")
    w = mixer.MixerWeights(*(lay[k].cuda() for k in workloads.MIXER_KEYS))
    h = lay["hidden"].cuda()
    stream = torch.cuda.current_stream()
    gemm_flops = 2.0 * b * L * (2 * d * dm + d * (r + 2 * n) + d * r + dm * d)
    if kind == "m1":
        ws = torch.empty(mixer.workspace_bytes(b, L, dm, d, n, r, torch.bfloat16), dtype=torch.uint8, device="cuda")
        out = torch.empty(b, L, dm, dtype=torch.bfloat16, device="cuda")

        def run(i):
            mixer.mixer_fwd(h, w, out=out, workspace=ws)
    else:
        ws = torch.empty(mixer.step_workspace_bytes(b, dm, d, n, r, torch.bfloat16), dtype=torch.uint8, device="cuda")
        out = torch.empty(b, dm, dtype=torch.bfloat16, device="cuda")
        cs = [torch.zeros(b, d, 3, device="cuda") for _ in range(2)]
        ss = [torch.zeros(b, d, n, device="cuda") for _ in range(2)]
        h1 = h[:, 0].contiguous()

        def run(i):
            mixer.mixer_step(h1, w, cs[i % 2], ss[i % 2], inplace=True, out=out, workspace=ws)
    ms_step = timed(run, steps, warmup, stream)
    graph_ms = None
    if kind == "m4":
        # the same decode step captured once in a HIP graph and replayed
        # (host launch overhead removed); states ping-pong as above
        g = [torch.cuda.CUDAGraph() for _ in range(2)]
        torch.cuda.synchronize()
        for i in range(2):
            with torch.cuda.graph(g[i]):
                run(i)
        torch.cuda.synchronize()
        graph_ms = timed(lambda i: g[i % 2].replay(), steps, warmup, stream)
    t = ms_step * 1e-3
    return dict(workload="mamba130m_mixer_layer_%s_b%d_l%d" % ("prefill" if kind == "m1" else "decode", b, L),
                graph_replay_ms=graph_ms,
                batch=b, seqlen=L, d_model=dm, d_inner=d, d_state=n, dt_rank=r, io_dtype="bf16",
                ms_per_step=ms_step, tokens_per_s=b * L / t, elems_per_s=b * L * d / t,
                gemm_tflops=gemm_flops / t / 1e12)


def bench_backward(steps, warmup):
    """Backward of the 130M-class prefill (batch 8 x 2048 tokens, d_inner 1536,
    d_state 16, bf16 io): mamba_scan_bwd, all gradients, with a preallocated
    workspace. Algorithmic bytes: x, dt, z, dy, B, C read; dx, ddt, dz (io) and
    dB, dC (float32) written; parameters and their gradients."""
    import torch
    import selective_state_space_07_amd as ms
    import workloads
    b, L, d, n = 8, 2048, 1536, 16
    lay = {k: v.cuda() for k, v in workloads.make_layer(b, L, d, n, torch.bfloat16, seed=23, params="config").items()}
    g = torch.Generator().manual_seed(24)
    dy = torch.randn(b, L, d, generator=g).to(torch.bfloat16).cuda()
    p = ms.Params(*(lay[k] for k in ("conv_w", "conv_b", "dt_bias", "D", "A")))
    ws = torch.empty(ms.mamba_scan_bwd_workspace_bytes(b, L, d, n, ms.MAMBA_BF16), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()

    def run(i):
        ms.bwd(lay["x"], lay["dt"], lay["z"], lay["B"], lay["C"], p, dy, workspace=ws)
    ms_step = timed(run, steps, warmup, stream)
    t = ms_step * 1e-3
    bld, bln = b * L * d * 2, b * L * n * 2
    alg = 7 * bld + 2 * bln + 2 * b * L * n * 4 + 2 * d * (4 + 3 + n) * 4
    slots = algorithmic_slots_bwd(n) * b * L * d
    # the training pair that keeps the forward's states: mamba_scan_fwd_ckpt,
    # then mamba_scan_bwd_ckpt (the backward without its own forward pass),
    # against the plain prefill of the same inputs
    ck = ms.ckpt_like(lay["x"])
    y = torch.empty_like(lay["x"])
    ws2 = torch.empty(ms.mamba_scan_bwd_ckpt_workspace_bytes(b, L, d, n, ms.MAMBA_BF16), dtype=torch.uint8,
                      device="cuda")

    def run_fwd(i):
        ms.fwd(lay["x"], lay["dt"], lay["z"], lay["B"], lay["C"], p, out=y, return_states=False)

    def run_fwd_ckpt(i):
        ms.fwd(lay["x"], lay["dt"], lay["z"], lay["B"], lay["C"], p, out=y, return_states=False, ckpt=ck)

    def run_bwd_ckpt(i):
        ms.bwd(lay["x"], lay["dt"], lay["z"], lay["B"], lay["C"], p, dy, workspace=ws2, ckpt=ck)
    fwd_ms = timed(run_fwd, steps, warmup, stream)
    fwd_ckpt_ms = timed(run_fwd_ckpt, steps, warmup, stream)
    bwd_ckpt_ms = timed(run_bwd_ckpt, steps, warmup, stream)
    return dict(workload="mamba130m_scan_backward_b%d_l%d_d%d_n%d_bf16" % (b, L, d, n), batch=b, seqlen=L,
                d_inner=d, d_state=n, io_dtype="bf16", ms_per_step=ms_step, elems_per_s=b * L * d / t,
                alg_bytes=alg, hbm_gbs=alg / t / 1e9, hbm_frac=alg / t / 1e9 / PEAK_HBM_GBS,
                alg_valu_slots=slots, valu_gslots=slots / t / 1e9, valu_frac=slots / t / 1e9 / PEAK_VALU_GSLOTS,
                train_step=dict(fwd_ms=fwd_ms, bwd_ms=ms_step, fwd_ckpt_ms=fwd_ckpt_ms, bwd_from_ckpt_ms=bwd_ckpt_ms,
                                recompute_pair_ms=fwd_ms + ms_step, ckpt_pair_ms=fwd_ckpt_ms + bwd_ckpt_ms))


def bench_ssd(steps, warmup):
    """Mamba-2 SSD scan of a Foundation-V3-like layer (d_inner 1536 as 24 heads
    of 64, d_state 128, one group) over batch 8 x 2048 tokens, bf16 io, with a
    preallocated workspace. Algorithmic work: the chunked form's products, each
    counted once (C B^T per chunk and group, the causal half of G x, the chunk
    state and the carried-state readout per head); algorithmic bytes: x, dt, B,
    C read, y written, parameters, final state."""
    import torch
    import selective_state_space_07_amd as ms
    import workloads
    b, L, H, P, N, G = 8, 2048, 24, 64, 128, 1
    lay = {k: v.cuda() for k, v in workloads.make_ssd(b, L, H, P, N, G, torch.bfloat16, seed=29, params="config").items()}
    ws = torch.empty(ms.ssd_workspace_bytes(b, L, H, P, N, G, torch.bfloat16), dtype=torch.uint8, device="cuda")
    y = torch.empty_like(lay["x"])
    so = torch.empty(b, H, P, N, device="cuda")
    stream = torch.cuda.current_stream()

    def run(i):
        ms.ssd_fwd(*(lay[k] for k in workloads.SSD_KEYS), out=y, state_out=so, workspace=ws)
    ms_step = timed(run, steps, warmup, stream)
    t = ms_step * 1e-3
    Q = 256
    chunks = b * ((L + Q - 1) // Q)
    flops = chunks * (G * 2.0 * Q * Q * N + H * (Q * Q * P + 2.0 * Q * N * P + 2.0 * Q * N * P))
    alg = b * L * (2 * H * P + H + 2 * G * N) * 2 + 3 * H * 4 + b * H * P * N * 4
    return dict(workload="mamba2_ssd_b%d_l%d_h%d_p%d_n%d_bf16" % (b, L, H, P, N), batch=b, seqlen=L, nheads=H,
                headdim=P, d_state=N, io_dtype="bf16", ms_per_step=ms_step, tokens_per_s=b * L / t,
                elems_per_s=b * L * H * P / t, alg_flops=flops, tflops=flops / t / 1e12,
                mfma_frac=flops / t / 1e12 / PEAK_BF16_TFLOPS, alg_bytes=alg, hbm_gbs=alg / t / 1e9,
                hbm_frac=alg / t / 1e9 / PEAK_HBM_GBS)


def bench_ssd_step(steps, warmup):
    """One Mamba-2 SSD decode token (mamba2_ssd_step) for batch 256 of the same
    layer (24 heads of 64, d_state 128, bf16 io, float32 state updated in place,
    two state buffers alternating). Memory-bound: algorithmic bytes = the state
    read and written, plus the token's inputs and output."""
    import torch
    import selective_state_space_07_amd as ms
    import workloads
    b, H, P, N = 256, 24, 64, 128
    lay = {k: v.cuda() for k, v in workloads.make_ssd(b, 1, H, P, N, 1, torch.bfloat16, seed=37, params="config").items()}
    x, dt, B, C = (lay[k][:, 0].contiguous() for k in ("x", "dt", "B", "C"))
    st = [torch.zeros(b, H, P, N, device="cuda") for _ in range(2)]
    y = torch.empty_like(x)
    stream = torch.cuda.current_stream()

    def run(i):
        ms.ssd_step(x, dt, B, C, lay["dt_bias"], lay["A"], lay["D"], st[i % 2], inplace=True, out=y)
    ms_step = timed(run, steps, warmup, stream)
    t = ms_step * 1e-3
    alg = 2 * b * H * P * N * 4 + 2 * b * H * P * 2 + b * H * 2 + 2 * b * N * 2 + 3 * H * 4
    copy_gbs = copy_rate(alg, 1, steps, warmup, stream)
    return dict(workload="mamba2_ssd_decode_b%d_h%d_p%d_n%d_bf16" % (b, H, P, N), batch=b, nheads=H, headdim=P,
                d_state=N, io_dtype="bf16", ms_per_step=ms_step, tokens_per_s=b / t, alg_bytes=alg,
                hbm_gbs=alg / t / 1e9, hbm_frac=alg / t / 1e9 / PEAK_HBM_GBS, copy_same_size_gbs=copy_gbs,
                frac_of_copy=alg / t / 1e9 / copy_gbs)


def cpu_baseline(index, seconds):
    """The fp64 oracle as it stands, timed on this host's cores over whole
    repetitions of the workload until `seconds` have passed."""
    import oracle
    import workloads
    cfg = workloads.WORKLOADS[index]
    lay = workloads.make_config(index)
    cores = len(os.sched_getaffinity(0))
    env = os.environ.get("OMP_NUM_THREADS")
    if env and env.isdigit():
        cores = min(cores, int(env))
    args = [lay[k] for k in ("x", "dt", "z", "B", "C", "conv_w", "conv_b", "dt_bias", "D", "A")]
    import numpy as np
    f64 = [np.ascontiguousarray(a.double().numpy()) for a in args]
    reps, t_total = 0, 0.0
    while t_total < seconds:
        t0 = time.perf_counter()
        oracle.oracle_fwd(*f64, nthreads=cores)
        t_total += time.perf_counter() - t0
        reps += 1
    elems = cfg["batch"] * cfg["seqlen"] * cfg["d_inner"] * reps
    one_thread = {}
    for i in (0, 1, 2):  # the same oracle on one thread, one call per workload
        c = workloads.WORKLOADS[i]
        lay_i = workloads.make_config(i)
        a_i = [np.ascontiguousarray(lay_i[k].double().numpy()) for k in
               ("x", "dt", "z", "B", "C", "conv_w", "conv_b", "dt_bias", "D", "A")]
        t0 = time.perf_counter()
        oracle.oracle_fwd(*a_i, nthreads=1)
        dt_ = time.perf_counter() - t0
        one_thread[c["name"]] = dict(seconds=dt_, elems_per_s=c["batch"] * c["seqlen"] * c["d_inner"] / dt_)
    return dict(value=elems / t_total, unit="elems/s", cores=cores, kind="oracle",
                sample="%d x the whole workload (%dx%dx%d, d_state %d), fp64 sequential oracle, OpenMP over (b,d)"
                % (reps, cfg["batch"], cfg["seqlen"], cfg["d_inner"], cfg["d_state"]), seconds=t_total,
                cpu_model=cpu_model(), one_thread=one_thread)


def cpu_model():
    """The host CPU's model name (/proc/cpuinfo), or None."""
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


# Instructions per lane and round of each probe kind: (VALU, of which transcendental).
PROBE_KINDS = {0: ("fma_independent", 32, 0), 1: ("exp2_independent", 32, 32), 2: ("exp2_1_per_3_fma", 32, 8),
               3: ("fma_dependent_chain", 32, 0), 4: ("log2_plus_add", 64, 32), 5: ("rcp_plus_add", 64, 32),
               6: ("mul_dpp_row_bcast", 32, 0), 7: ("mul_plain", 32, 0), 8: ("v_add_f32_e32", 32, 0),
               9: ("v_fmac_f32_e32", 32, 0), 10: ("v_fma_f32_vop3_vgprs", 32, 0), 11: ("v_mul_f32_e64", 32, 0),
               12: ("v_mul_f32_e32", 32, 0), 13: ("exp2_1_per_3_mul", 32, 8)}


def valu_probe(waves=(1, 2, 3, 4, 8), iters=4096):
    """Issue rate of plain fp32 VALU and transcendental instructions on this
    GPU, against the 16-lanes-per-SIMD rate at the measured shader clock."""
    import ctypes
    from selective_state_space_07_amd import build as lib_build
    lib = ctypes.CDLL(lib_build.PROBE_LIB)
    lib.mamba_probe_valu.restype = ctypes.c_int
    lib.mamba_probe_valu.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.POINTER(ctypes.c_float),
                                     ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_longlong),
                                     ctypes.POINTER(ctypes.c_longlong), ctypes.POINTER(ctypes.c_int32)]
    import torch
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    rows = []
    for kind, (name, instr, trans) in PROBE_KINDS.items():
        for w in waves:
            ms_, ops = ctypes.c_float(), ctypes.c_double()
            st, wt, rate = ctypes.c_longlong(), ctypes.c_longlong(), ctypes.c_int32()
            rc = lib.mamba_probe_valu(kind, w, iters, ctypes.byref(ms_), ctypes.byref(ops), ctypes.byref(st),
                                      ctypes.byref(wt), ctypes.byref(rate))
            if rc != 0:
                raise SystemExit("probe kind %d failed: %d" % (kind, rc))
            t = ms_.value * 1e-3
            clk_ghz = st.value / (wt.value / (rate.value * 1e3)) / 1e9 if wt.value > 0 else None
            lanes = cus * w * 256
            instr_total = lanes * iters * instr / 64.0  # wave instructions
            # a wave64 instruction occupies a 16-lane SIMD for 4 cycles at full rate
            per_simd_cycles = instr_total / (cus * 4) * 4
            frac = per_simd_cycles / (t * clk_ghz * 1e9) if clk_ghz else None
            rows.append(dict(kind=name, waves_per_simd=w, ms=ms_.value, wave_instructions=instr_total,
                             transcendental_per_round=trans, instructions_per_round=instr, shader_clock_ghz=clk_ghz,
                             issue_frac_at_clock=frac,
                             lane_ops_per_s=lanes * iters * instr / t,
                             issue_frac_at_2p4ghz=per_simd_cycles / (t * 2.4e9)))
    return dict(probe="valu_issue_rate", cus=cus, iters=iters, rows=rows)


def run_workload(tok, a):
    """One workload by its token: 0-4 (a trailing p: packed documents), m1 / m4, b1, s1 / s4."""
    if tok.startswith("m"):
        return bench_mixer(tok, a.steps, a.warmup)
    if tok == "b1":
        return bench_backward(a.steps, a.warmup)
    if tok == "s1":
        return bench_ssd(a.steps, a.warmup)
    if tok == "s4":
        return bench_ssd_step(a.steps, a.warmup)
    packed = tok.endswith("p")
    idx = int(tok[:-1] if packed else tok)
    if idx == 4:
        return bench_decode(a.steps, a.warmup)
    return bench_prefill(idx, a.steps, a.warmup, a.rotate_bytes, packed=packed)


def main():
    global WARM_SECONDS
    a = parse()
    WARM_SECONDS = max(0.0, a.warm_seconds)
    if a.pmc_summary:
        if a.copy_calib <= 0:
            raise SystemExit("--pmc-summary needs --copy-calib BYTES (the size the runs used)")
        calib = int(a.copy_calib) // 4 * 4
        counters = pmc_summary(a.pmc_summary[0], a.pmc_summary[1], calib)
        line = dict(counters=counters)
        if a.update_traffic:
            if a.only not in ("1", "4"):
                raise SystemExit("--update-traffic needs --only 1 or --only 4")
            line["recorded"] = update_traffic(int(a.only), counters, calib, a.kernel_stats)
        print(json.dumps(line))
        return
    if a.sq_summary:
        print(json.dumps(sq_summary(a.sq_summary, int(a.only or "1"))))
        return
    if a.valu_probe:
        import torch
        if not torch.cuda.is_available():
            raise SystemExit("no GPU visible")
        print(json.dumps(valu_probe()))
        return
    if a.gpus != 1:
        print("bench.py measures one GPU only: the selective-scan path is built and timed on a single "
              "MI355X (per-GPU shard); --gpus %d is not supported." % a.gpus, file=sys.stderr)
        sys.exit(2)
    import torch
    import selective_state_space_07_amd as ms
    ms.load()
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    if a.only is not None:
        # Profile mode (for rocprofv3): one workload, no CPU baseline, plain
        # timing line; optionally a calibration copy of known size first.
        if a.copy_calib > 0:
            n = int(a.copy_calib) // 4
            src = torch.full((n,), -1.0, device="cuda")
            dst = torch.empty_like(src)
            for _ in range(max(1, a.steps)):
                torch.abs(src, out=dst)
            torch.cuda.synchronize()
            print(json.dumps({"copy_calib_bytes_read": n * 4, "copy_calib_bytes_written": n * 4}))
        r = run_workload(a.only, a)
        print(json.dumps(r))
        return
    order = [s.strip() for s in a.workloads.split(",") if s.strip()]
    if not order or not order[0].isdigit():
        raise SystemExit("--workloads must start with the workload the line reports (0-4), got %r" % a.workloads)
    head = int(order[0])
    results = {}
    for tok in order:
        print("bench: workload %s" % tok, file=sys.stderr, flush=True)
        results[tok] = run_workload(tok, a)
    h = results[order[0]]
    cpu = None
    if not a.no_cpu_baseline and head != 4:
        print("bench: cpu baseline", file=sys.stderr, flush=True)
        cpu = cpu_baseline(head, a.cpu_seconds)
    tr = traffic_entry(head)
    traffic = None if tr is None else tr["fetch_bytes"] + tr["write_bytes"]
    if head == 4:
        roof = dict(bound="hbm", achieved=h["hbm_gbs"], peak=PEAK_HBM_GBS, unit="GB/s", frac=h["hbm_frac"],
                    traffic=None, kernel="scan_step_vec_kernel x24 (one decode step)")
    else:
        # per launch: the call's own device time (HIP events around each call),
        # not the call-to-call period of the timed loop (ms_per_step)
        roof = dict(bound="alu", achieved=h["launch_valu_gslots"], peak=PEAK_VALU_GSLOTS, unit="Gslot/s",
                    frac=h["launch_valu_frac"], traffic=traffic,
                    kernel=tr["kernel"] if tr else "all kernels of one prefill call",
                    alg_slots_per_launch=h["alg_valu_slots"], launch_us=h["launch_ms"] * 1e3,
                    call_period_us=h["ms_per_step"] * 1e3,
                    slot_pricing=dict(plain_ops_per_elem=algorithmic_ops(h["d_state"])[0],
                                      transcendentals_per_elem=algorithmic_ops(h["d_state"])[1],
                                      slots_per_transcendental=TRANS_SLOTS,
                                      peak_basis="fp32 vector 157.3 TFLOP/s / 2 flops per FMA"),
                    hbm=dict(achieved=h["launch_hbm_gbs"], peak=PEAK_HBM_GBS, unit="GB/s",
                             frac=h["launch_hbm_frac"], alg_bytes_per_launch=h["alg_bytes"]))
        if tr:
            roof["traffic_detail"] = tr
    line = {
        "metric": "scan B*L*d_inner elems/s + achieved HBM GB/s (% peak), prefill & decode step",
        "value": h["elems_per_s"], "unit": "elems/s", "n_gpus": 1, "steps": a.steps, "warmup": a.warmup, "warm_seconds": WARM_SECONDS,
        "ms_per_step": h["ms_per_step"], "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32", "data": "synthetic (seeded)",
        "config": {"workload": h["workload"], "batch": h["batch"], "seqlen": h.get("seqlen", 1),
                   "d_inner": h["d_inner"], "d_state": h["d_state"], "io_dtype": h["io_dtype"],
                   "state_dtype": "f32"},
        "hbm_gbs": h["hbm_gbs"], "hbm_frac": h["hbm_frac"],
        "roofline": roof, "cpu_baseline": cpu,
        "workloads": {str(k): v for k, v in results.items()},
        "device": torch.cuda.get_device_name(0), "library": ms.library_path(),
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
