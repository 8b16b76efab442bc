"""MI355X (gfx950) selective-scan mixer core behind the C ABI of libmamba_scan.

`fwd` (full-sequence prefill, optionally over packed documents), `bwd` (the
prefill's gradients), `step` (one-token decode) and `ssd_fwd` (the Mamba-2
SSD scan) take torch tensors
on the GPU and call the library's HIP kernels; PyTorch only provides device
memory and the stream. The raw C entry points are re-exported under their C
names. There is no fallback: without the library or a gfx950 device every
call raises MambaScanError.
"""
from ._binding import (EXPORTS, MAMBA_BF16, MAMBA_F32, MambaScanError, library_path, load,
                       mamba_scan_abi_version, mamba_scan_bwd, mamba_scan_bwd_ckpt,
                       mamba_scan_bwd_ckpt_workspace_bytes, mamba_scan_bwd_workspace_bytes, mamba_scan_ckpt_bytes,
                       mamba_scan_fwd_ckpt,
                       mamba_scan_call_count, mamba_scan_fwd, mamba_scan_fwd_seq, mamba_scan_fwd_workspace_bytes,
                       mamba2_ssd_fwd, mamba2_ssd_fwd_seq, mamba2_ssd_fwd_workspace_bytes, mamba2_ssd_step, mamba_scan_last_error, mamba_scan_status_str,
                       mamba_scan_step, mamba_scan_testing_fwd, mamba_scan_testing_fwd_workspace_bytes,
                       mamba_scan_fwd_noalloc, NOALLOC_SCRATCH_BYTES, mamba_scan_fwd_xc,
                       mamba_scan_step_xc, mamba_scan_step_xc_dtproj, mamba_scan_fwd_xc_dtproj)
from .api import Params, bwd, ckpt_like, fwd, step, workspace_bytes
from .ssd import ssd_fwd, ssd_step, ssd_workspace_bytes

__all__ = ["fwd", "bwd", "step", "ckpt_like", "mamba_scan_bwd_ckpt", "mamba_scan_bwd_ckpt_workspace_bytes",
           "mamba_scan_ckpt_bytes", "mamba_scan_fwd_ckpt", "ssd_fwd", "ssd_step", "ssd_workspace_bytes", "Params", "workspace_bytes", "MambaScanError", "MAMBA_F32", "MAMBA_BF16", "EXPORTS",
           "load", "library_path", "mamba_scan_abi_version", "mamba_scan_bwd", "mamba_scan_bwd_workspace_bytes",
           "mamba_scan_call_count", "mamba_scan_fwd",
           "mamba_scan_fwd_seq", "mamba_scan_fwd_workspace_bytes", "mamba2_ssd_fwd", "mamba2_ssd_fwd_seq", "mamba2_ssd_fwd_workspace_bytes", "mamba2_ssd_step", "mamba_scan_last_error", "mamba_scan_status_str", "mamba_scan_step",
           "mamba_scan_testing_fwd", "mamba_scan_testing_fwd_workspace_bytes", "mamba_scan_fwd_noalloc",
           "NOALLOC_SCRATCH_BYTES", "mamba_scan_fwd_xc",
           "mamba_scan_step_xc", "mamba_scan_step_xc_dtproj", "mamba_scan_fwd_xc_dtproj"]
