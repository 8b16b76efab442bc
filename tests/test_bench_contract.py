"""bench.py's output contract: one JSON line with the headline metric, its
roofline object and the CPU baseline; more than one GPU is refused with a
message (checked without a GPU)."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    out = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                         text=True, cwd=ROOT, timeout=120)
    assert out.returncode != 0
    assert "--gpus 2" in out.stderr, out.stderr
    assert out.stdout.strip() == ""


@pytest.mark.gpu
def test_json_line_contract():
    """A short default-shaped run: the headline workload and one more, with a
    one-second CPU baseline; checks the keys and their consistency."""
    out = subprocess.run([sys.executable, "-u", os.path.join(ROOT, "bench.py"), "--steps", "3", "--warmup", "1",
                          "--workloads", "1,0", "--cpu-seconds", "1"], capture_output=True, text=True, cwd=ROOT,
                         timeout=600)
    assert out.returncode == 0, out.stderr[-2000:]
    lines = [l for l in out.stdout.splitlines() if l.strip()]
    assert len(lines) == 1, out.stdout
    d = json.loads(lines[0])
    for k in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better", "scaling",
              "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline"):
        assert k in d, k
    assert d["n_gpus"] == 1 and d["steps"] == 3 and d["warmup"] == 1 and d["higher_is_better"] is True
    assert d["value"] > 0 and d["ms_per_step"] > 0
    assert "workload" in d["config"]
    r = d["roofline"]
    for k in ("bound", "achieved", "peak", "unit", "frac", "traffic"):
        assert k in r, k
    assert r["bound"] in ("hbm", "mfma", "alu")
    assert abs(r["frac"] - r["achieved"] / r["peak"]) < 1e-9
    assert 0 < r["frac"] < 1
    c = d["cpu_baseline"]
    assert c["kind"] == "oracle" and c["value"] > 0 and c["cores"] >= 1 and c["sample"]
