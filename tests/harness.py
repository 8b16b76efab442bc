"""Shared plumbing of the GPU tests: move a workload to the GPU, run the HIP
path through the package (hence the C ABI), and run the oracle on the same
values, optionally on a subset of channels."""
import numpy as np
import torch

import oracle
import selective_state_space_07_amd as ms

IO_KEYS = ("x", "dt", "z", "B", "C")
PARAM_KEYS = ("conv_w", "conv_b", "dt_bias", "D", "A")


def to_gpu(layer):
    return {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in layer.items()}


def params_of(layer):
    return ms.Params(*(layer[k] for k in PARAM_KEYS))


def gpu_fwd(layer, conv_state=None, ssm_state=None, **kw):
    """layer: dict of GPU tensors."""
    return ms.fwd(layer["x"], layer["dt"], layer["z"], layer["B"], layer["C"], params_of(layer), conv_state,
                  ssm_state, **kw)


def gpu_step(tok, params, conv_state, ssm_state, **kw):
    return ms.step(tok["x"], tok["dt"], tok["z"], tok["B"], tok["C"], params, conv_state, ssm_state, **kw)


def oracle_fwd(layer, conv_state=None, ssm_state=None, channels=None, nthreads=0):
    """Run the oracle on (a channel subset of) a layer. Returns float64 arrays
    restricted to `channels` along d."""
    cpu = {k: v.detach().cpu() for k, v in layer.items()}
    cs = None if conv_state is None else conv_state.detach().cpu()
    ss = None if ssm_state is None else ssm_state.detach().cpu()
    if channels is not None:
        idx = torch.as_tensor(channels)
        for k in ("x", "dt", "z"):
            cpu[k] = cpu[k][..., idx].contiguous()
        for k in PARAM_KEYS:
            cpu[k] = cpu[k][idx].contiguous()
        cs = None if cs is None else cs[:, idx].contiguous()
        ss = None if ss is None else ss[:, idx].contiguous()
    return oracle.oracle_fwd(*(cpu[k] for k in IO_KEYS + PARAM_KEYS), cs, ss, nthreads=nthreads)


def oracle_step(tok, params_cpu, conv_state, ssm_state, channels=None, states_sliced=False):
    """One oracle step on (a channel subset of) a layer. With `states_sliced`
    the given states already hold only `channels` (float64 kept as is)."""
    t = {k: v.detach().cpu() for k, v in tok.items()}
    p = {k: v.detach().cpu() for k, v in params_cpu.items()}
    cs, ss = conv_state.detach().cpu(), ssm_state.detach().cpu()
    if channels is not None:
        idx = torch.as_tensor(channels)
        for k in ("x", "dt", "z"):
            t[k] = t[k][:, idx].contiguous()
        for k in PARAM_KEYS:
            p[k] = p[k][idx].contiguous()
        if not states_sliced:
            cs, ss = cs[:, idx].contiguous(), ss[:, idx].contiguous()
    return oracle.oracle_step(*(t[k] for k in IO_KEYS), *(p[k] for k in PARAM_KEYS), cs, ss)


def cols(a, channels, axis):
    """Select `channels` along `axis` of a torch tensor (on the CPU)."""
    a = a.detach().cpu()
    if channels is None:
        return a
    return a.index_select(axis, torch.as_tensor(channels))
