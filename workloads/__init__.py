"""Seeded synthetic inputs for the selective-scan mixer core.

This module only draws numbers: it holds none of the method's arithmetic and is
shared by the tests, the smoke check and the benchmark. Both the HIP path and
the oracle consume the exact tensors it returns (io values already rounded to
their dtype, parameters in float32).

Recipe of the five workloads (params="config"):
  A_log[d, n] = log(n + 1), A = -exp(A_log) computed in float64 and rounded to
  float32 (so A[d, n] = -(n + 1) exactly); D = 1; conv_w ~ U(-0.5, 0.5);
  conv_b = 0; dt_bias = softplus^-1(u) with u log-uniform in `dt_range`;
  x, z, B, C ~ N(0, 1); dt (the projection output without bias) ~ 0.1 * N(0, 1).
  Draw order: conv_w, u (for dt_bias), x, z, dt, B, C from
  numpy.random.Generator(PCG64(seed)). Values are drawn in float32 (float64 for
  the uniforms) and cast to the io dtype with torch (round to nearest even).

Parameters drawn per channel (params="random", the default of make_layer and
the other layer generators): after the draws above, from the same generator,
A[d, n] = -U(0.5, 8) independently for every (d, n), D[d] = 1 + 0.5 * N(0, 1),
conv_b[d] = 0.1 * N(0, 1) (all rounded to float32). The recurrence is per
(d, n) in A and per d in D and the conv bias, and parameters that vary along
both indices make a kernel that reads the wrong index disagree with the oracle.
"""
import math

import numpy as np
import torch

# The five workloads: shapes and dtypes of the pages' workloads (CALM nano-like
# tiny prefill; a 130M-class Mamba layer; a wide short "large"-profile prefill;
# a long-context prefill; a 24-layer decode step with states from a 128-token
# prefill).
WORKLOADS = [
    dict(index=0, name="tiny_fp32_prefill_b2_l64_d128_n16", kind="prefill", batch=2, seqlen=64, d_inner=128,
         d_state=16, dtype=torch.float32, dt_range=(1e-3, 1e-1)),
    dict(index=1, name="mamba130m_bf16_prefill_b8_l2048_d1536_n16", kind="prefill", batch=8, seqlen=2048,
         d_inner=1536, d_state=16, dtype=torch.bfloat16, dt_range=(1e-3, 1e-1)),
    dict(index=2, name="wide_fp32_prefill_b16_l64_d2048_n8", kind="prefill", batch=16, seqlen=64, d_inner=2048,
         d_state=8, dtype=torch.float32, dt_range=(1e-3, 1e-1)),
    dict(index=3, name="long_bf16_prefill_b1_l65536_d1536_n16", kind="prefill", batch=1, seqlen=65536,
         d_inner=1536, d_state=16, dtype=torch.bfloat16, dt_range=(1e-4, 1e-1)),
    dict(index=4, name="decode_bf16_24x_b256_d1536_n16", kind="decode", batch=256, layers=24, prefill_len=128,
         d_inner=1536, d_state=16, dtype=torch.bfloat16, dt_range=(1e-3, 1e-1)),
]

BASE_SEED = 7000


def _softplus_inv(u):
    # inverse of log(1 + e^v): v = log(e^u - 1), in float64
    return np.log(np.expm1(u))


def _check_params(params):
    if params not in ("config", "random"):
        raise ValueError("params must be 'config' or 'random', not %r" % (params,))


def make_layer(batch, seqlen, d_inner, d_state, dtype=torch.float32, seed=0, dt_range=(1e-3, 1e-1), d_conv=4,
               params="random"):
    """Draw one layer's inputs. Returns a dict of CPU torch tensors:
    x, dt, z [batch, seqlen, d_inner] and B, C [batch, seqlen, d_state] in `dtype`;
    conv_w [d_inner, d_conv], conv_b, dt_bias, D [d_inner], A [d_inner, d_state] in float32.
    `seed` may be an int or a numpy SeedSequence. `params` = "config" keeps the
    workloads' A, D and conv_b; "random" draws them per channel (see above)."""
    _check_params(params)
    rng = np.random.Generator(np.random.PCG64(seed))
    A_log = np.log(np.arange(1, d_state + 1, dtype=np.float64))[None, :].repeat(d_inner, 0)
    A = (-np.exp(A_log)).astype(np.float32)
    Dp = np.ones(d_inner, dtype=np.float32)
    conv_w = rng.uniform(-0.5, 0.5, size=(d_inner, d_conv)).astype(np.float32)
    conv_b = np.zeros(d_inner, dtype=np.float32)
    lo, hi = math.log(dt_range[0]), math.log(dt_range[1])
    u = np.exp(rng.uniform(lo, hi, size=d_inner))
    dt_bias = _softplus_inv(u).astype(np.float32)
    x = rng.standard_normal((batch, seqlen, d_inner), dtype=np.float32)
    z = rng.standard_normal((batch, seqlen, d_inner), dtype=np.float32)
    dt = rng.standard_normal((batch, seqlen, d_inner), dtype=np.float32) * np.float32(0.1)
    B = rng.standard_normal((batch, seqlen, d_state), dtype=np.float32)
    C = rng.standard_normal((batch, seqlen, d_state), dtype=np.float32)
    if params == "random":
        A, Dp, conv_b = _random_params(rng, d_inner, d_state)
    t = lambda a: torch.from_numpy(a)
    io = lambda a: torch.from_numpy(a).to(dtype)
    return dict(x=io(x), dt=io(dt), z=io(z), B=io(B), C=io(C), conv_w=t(conv_w), conv_b=t(conv_b),
                dt_bias=t(dt_bias), D=t(Dp), A=t(A))


def _random_params(rng, d_inner, d_state):
    """A [d_inner, d_state] = -U(0.5, 8), D [d_inner] = 1 + 0.5 N(0, 1),
    conv_b [d_inner] = 0.1 N(0, 1), float32, in that draw order."""
    A = (-rng.uniform(0.5, 8.0, size=(d_inner, d_state))).astype(np.float32)
    Dp = (1.0 + 0.5 * rng.standard_normal(d_inner)).astype(np.float32)
    conv_b = (0.1 * rng.standard_normal(d_inner)).astype(np.float32)
    return A, Dp, conv_b


def make_config(index, seqlen=None, batch=None):
    """Inputs of prefill workload `index` (0-3), optionally with a shorter
    sequence or smaller batch drawn from the same seed (a prefix sample is NOT
    implied: a different shape is a different draw)."""
    cfg = WORKLOADS[index]
    assert cfg["kind"] == "prefill"
    return make_layer(batch or cfg["batch"], seqlen or cfg["seqlen"], cfg["d_inner"], cfg["d_state"], cfg["dtype"],
                      seed=BASE_SEED + index, dt_range=cfg["dt_range"], params="config")


def make_decode_layers(layers=None, batch=None, prefill_len=None, d_inner=None):
    """Workload 4: per layer l, an independent draw (SeedSequence(7004).spawn)
    of parameters and prefill_len + 1 tokens. Returns a list of dicts, each with
    'prefill' (the first prefill_len tokens, [batch, prefill_len, ...]) and
    'token' (the last token, [batch, ...]) plus the parameters."""
    cfg = WORKLOADS[4]
    layers = layers or cfg["layers"]
    batch = batch or cfg["batch"]
    prefill_len = prefill_len or cfg["prefill_len"]
    d_inner = d_inner or cfg["d_inner"]
    seeds = np.random.SeedSequence(BASE_SEED + 4).spawn(layers)
    out = []
    for s in seeds:
        lay = make_layer(batch, prefill_len + 1, d_inner, cfg["d_state"], cfg["dtype"], seed=s,
                         dt_range=cfg["dt_range"], params="config")
        pre = {k: lay[k][:, :prefill_len].contiguous() for k in ("x", "dt", "z", "B", "C")}
        tok = {k: lay[k][:, prefill_len].contiguous() for k in ("x", "dt", "z", "B", "C")}
        params = {k: lay[k] for k in ("conv_w", "conv_b", "dt_bias", "D", "A")}
        out.append(dict(prefill=pre, token=tok, params=params))
    return out


def sample_channels(d_inner, count, seed):
    """Sorted distinct channel indices for sampled full-size checks (always
    includes the first and last channel)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    idx = set(rng.choice(d_inner, size=min(count, d_inner), replace=False).tolist())
    idx.update({0, d_inner - 1})
    return np.array(sorted(idx))


# Packed-document layouts (document ids along t, per batch row) covering the
# structural cases the niverel-mamba page certifies for seq_idx strict reset:
# boundary at position 0, length-1 documents, consecutive boundaries, a
# boundary on a block edge, a document inside one block, boundaries that differ
# across batch rows, terminal padding, a non-zero first id, many short
# documents (ids may repeat: every change of id starts a new document).
SEQ_CASES = ("boundary_at_0", "length_1_docs", "consecutive_boundaries", "boundary_on_edge", "doc_inside_block",
             "misaligned_rows", "terminal_padding", "nonzero_first_id", "many_short_docs")


def make_seq_idx(case, batch, seqlen, edge=16, seed=0):
    """int32 [batch, seqlen] document ids for one of SEQ_CASES. `edge` is the
    block length whose edges the boundary cases align to (or avoid)."""
    L = seqlen
    rng = np.random.default_rng(seed)
    ids = np.zeros((batch, L), dtype=np.int32)
    for b in range(batch):
        r = ids[b]
        if case == "boundary_at_0":          # a length-1 document at t = 0, then one more
            r[1:] = 1
        elif case == "length_1_docs":        # length-1 documents in the middle and at the end
            m = L // 2
            r[m:] = 1
            if m + 1 < L:
                r[m + 1:] = 2
            if m + 2 < L:
                r[m + 2:] = 3
            r[L - 1] = 4
        elif case == "consecutive_boundaries":  # a run of changes at consecutive steps
            s = max(1, L // 3)
            for k, t in enumerate(range(s, min(L, s + 6))):
                r[t:] = k + 1
        elif case == "boundary_on_edge":     # changes exactly at block edges
            for k, t in enumerate(range(edge, L, edge)):
                if k % 2 == 0:
                    r[t:] = k + 1
        elif case == "doc_inside_block":     # a short document strictly inside one block
            s = edge + edge // 4
            e = min(L, s + max(1, edge // 2))
            if s < L:
                r[s:e] = 1
                r[e:] = 2
        elif case == "misaligned_rows":      # boundaries at different places per row
            cut = int(rng.integers(1, max(2, L)))
            r[cut:] = 1
            cut2 = int(rng.integers(cut, L + 1))
            r[cut2:] = 2
        elif case == "terminal_padding":     # trailing padding with its own id
            pad = max(1, L // 5)
            r[:] = 3
            r[L - pad:] = -1
        elif case == "nonzero_first_id":
            r[:] = 7
            r[L // 2:] = 9
        elif case == "many_short_docs":      # lengths 1..4, ids alternating (repeats start new documents)
            t, k = 0, 0
            while t < L:
                n = int(rng.integers(1, 5))
                r[t:t + n] = k % 2
                t += n
                k += 1
        else:
            raise ValueError(case)
    return ids


def segments(ids_row):
    """[start, end) of each document of one row: maximal runs of equal ids."""
    cuts = [0] + [t for t in range(1, len(ids_row)) if ids_row[t] != ids_row[t - 1]] + [len(ids_row)]
    return list(zip(cuts[:-1], cuts[1:]))


def make_mixer_layer(batch, seqlen, d_model, d_inner, d_state, dt_rank, dtype=torch.float32, seed=0,
                     dt_range=(1e-3, 1e-1), conv_bias=0.0, params="random"):
    """Inputs and weights of one whole mixer layer (in_proj, conv, x_proj,
    dt_proj, scan, gate, out_proj). Weights ~ U(-1/sqrt(fan_in), 1/sqrt(fan_in))
    in the torch Linear layout [out, in], rounded to `dtype`; hidden ~ N(0, 1);
    conv_w, dt_bias as in make_layer; conv_b ~ conv_bias * N(0, 1). A and D:
    the workloads' (A = -(n + 1), D = 1) with params="config"; with "random",
    A[d, n] = -U(0.5, 8) and D = 1 + 0.5 N(0, 1), drawn last.
    Draw order: w_in, conv_w, w_x, w_dt, u (for dt_bias), hidden, conv_b (, A, D)."""
    _check_params(params)
    rng = np.random.Generator(np.random.PCG64(seed))

    def lin(out_f, in_f):
        b = 1.0 / math.sqrt(in_f)
        return rng.uniform(-b, b, size=(out_f, in_f)).astype(np.float32)

    w_in = lin(2 * d_inner, d_model)
    conv_w = rng.uniform(-0.5, 0.5, size=(d_inner, 4)).astype(np.float32)
    w_x = lin(dt_rank + 2 * d_state, d_inner)
    w_dt = lin(d_inner, dt_rank)
    w_out = lin(d_model, d_inner)
    lo, hi = math.log(dt_range[0]), math.log(dt_range[1])
    u = np.exp(rng.uniform(lo, hi, size=d_inner))
    dt_bias = _softplus_inv(u).astype(np.float32)
    hidden = rng.standard_normal((batch, seqlen, d_model), dtype=np.float32)
    conv_b = (conv_bias * rng.standard_normal(d_inner)).astype(np.float32)
    A = (-np.exp(np.log(np.arange(1, d_state + 1, dtype=np.float64))[None, :].repeat(d_inner, 0))).astype(np.float32)
    Dp = np.ones(d_inner, dtype=np.float32)
    if params == "random":
        A = (-rng.uniform(0.5, 8.0, size=(d_inner, d_state))).astype(np.float32)
        Dp = (1.0 + 0.5 * rng.standard_normal(d_inner)).astype(np.float32)
    t = lambda a: torch.from_numpy(a)
    io = lambda a: torch.from_numpy(a).to(dtype)
    return dict(hidden=io(hidden), w_in=io(w_in), conv_w=t(conv_w), conv_b=t(conv_b), w_x=io(w_x), w_dt=io(w_dt),
                dt_bias=t(dt_bias), A=t(A), D=t(Dp), w_out=io(w_out))


MIXER_KEYS = ("w_in", "conv_w", "conv_b", "w_x", "w_dt", "dt_bias", "A", "D", "w_out")


# Mamba-2 SSD scan (the Foundation-V3-like configuration: d_inner 1536 as 24
# heads of headdim 64, d_state 128, one group of B/C shared by all heads).
SSD_KEYS = ("x", "dt", "B", "C", "dt_bias", "A", "D")


def make_ssd(batch, seqlen, nheads=24, headdim=64, d_state=128, ngroups=1, dtype=torch.bfloat16, seed=0,
             dt_range=(1e-3, 1e-1), a_range=(1.0, 16.0), params="random"):
    """Draw one SSD layer's inputs. Returns a dict of CPU torch tensors:
    x [batch, seqlen, nheads, headdim], dt [batch, seqlen, nheads], B, C
    [batch, seqlen, ngroups, d_state] in `dtype`; dt_bias, A, D [nheads] in
    float32. Recipe: A_log[h] = log(U(a_range)), A = -exp(A_log) rounded to
    float32; dt_bias = softplus^-1(u), u log-uniform in `dt_range`; D = 1
    (params="config") or D[h] = 1 + 0.5 N(0, 1) drawn last (params="random");
    x, B, C ~ N(0, 1); dt ~ 0.1 N(0, 1). Draw order: A_log, u, x, dt, B, C (, D)."""
    _check_params(params)
    rng = np.random.Generator(np.random.PCG64(seed))
    A = (-np.exp(np.log(rng.uniform(a_range[0], a_range[1], size=nheads)))).astype(np.float32)
    lo, hi = math.log(dt_range[0]), math.log(dt_range[1])
    dt_bias = _softplus_inv(np.exp(rng.uniform(lo, hi, size=nheads))).astype(np.float32)
    Dp = np.ones(nheads, dtype=np.float32)
    x = rng.standard_normal((batch, seqlen, nheads, headdim), dtype=np.float32)
    dt = rng.standard_normal((batch, seqlen, nheads), dtype=np.float32) * np.float32(0.1)
    B = rng.standard_normal((batch, seqlen, ngroups, d_state), dtype=np.float32)
    C = rng.standard_normal((batch, seqlen, ngroups, d_state), dtype=np.float32)
    if params == "random":
        Dp = (1.0 + 0.5 * rng.standard_normal(nheads)).astype(np.float32)
    io = lambda a: torch.from_numpy(a).to(dtype)
    t = lambda a: torch.from_numpy(a)
    return dict(x=io(x), dt=io(dt), B=io(B), C=io(C), dt_bias=t(dt_bias), A=t(A), D=t(Dp))
