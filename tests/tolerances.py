"""Sealed agreement rule between the HIP path and the fp64 oracle.

Per element: |got - want| <= rtol * max(|want|, rms(want)), with rtol = 1e-4
for float32 io and 2e-2 for bfloat16 io (applied to y and to the SSM state;
the state is always float32 but inherits the io dtype's rtol because it is
driven by io-rounded inputs and shares the output's error budget). The RMS
floor keeps values near a zero crossing from demanding more than the array's
scale allows. The conv state must match bit for bit. The rule is observed and
then sealed: widening it to make a test pass is a finding, not a fix.
"""
import numpy as np
import torch

RTOL = {torch.float32: 1e-4, torch.bfloat16: 2e-2}


def to_f64(a):
    if isinstance(a, torch.Tensor):
        return a.detach().cpu().double().numpy()
    return np.asarray(a, dtype=np.float64)


def stats(got, want):
    """Agreement statistics of two arrays (float64)."""
    g, w = to_f64(got).ravel(), to_f64(want).ravel()
    if g.size == 0:
        return dict(max_abs=0.0, max_scaled=0.0, rel_l2=0.0, cosine=1.0, rms=0.0, finite=True)
    rms = float(np.sqrt(np.mean(w * w)))
    scale = np.maximum(np.abs(w), rms)
    scale[scale == 0] = 1.0
    err = np.abs(g - w)
    nw = float(np.linalg.norm(w))
    return dict(max_abs=float(err.max()), max_scaled=float((err / scale).max()),
                rel_l2=float(np.linalg.norm(g - w) / nw) if nw > 0 else float(np.linalg.norm(g)),
                cosine=float(g @ w / (np.linalg.norm(g) * nw)) if nw > 0 and np.linalg.norm(g) > 0 else 1.0,
                rms=rms, finite=bool(np.all(np.isfinite(g))))


def within(got, want, rtol):
    s = stats(got, want)
    return s["finite"] and s["max_scaled"] <= rtol, s


def assert_close(got, want, rtol, what=""):
    ok, s = within(got, want, rtol)
    assert ok, "%s outside rtol %.1e: %s" % (what, rtol, s)
    return s


def assert_bitwise(got, want, what=""):
    """float32 bit patterns equal (`want` may be a float64 copy of float32 values)."""
    g = to_f64(got).astype(np.float32).view(np.uint32)
    w = to_f64(want).astype(np.float32).view(np.uint32)
    assert g.shape == w.shape, (what, g.shape, w.shape)
    same = g == w
    assert same.all(), "%s differs bitwise at %d elements" % (what, int((~same).sum()))
