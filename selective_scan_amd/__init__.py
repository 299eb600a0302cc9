"""MI355X (gfx950) selective state-space scan.

Python binding of the C ABI in ``include/ssm_scan.h`` (library ``libssm_scan.so``,
built in-tree by ``python -m selective_scan_amd.build``). The functions keep the
C names, take torch tensors that already live on the GPU, allocate outputs and
workspace with ``torch.empty`` and pass raw device pointers and the current HIP
stream. Every step of the computation runs in the library's HIP kernels; there
is no fallback of any kind: without the built library importing the low-level
module raises.
"""
from .ops import (  # noqa: F401
    SsmError,
    lib,
    ssm_diag_copy,
    ssm_diag_stream_scale,
    ssm_diag_valu_rate,
    ssm_scan3_fwd,
    ssm_scan3_workspace_size,
    ssm_step3,
    ssm_scan_bwd,
    ssm_scan_bwd_workspace_size,
    ssm_scan_fwd,
    ssm_scan_fwd_ex,
    ssm_scan_fwd_noalloc,
    ssm_scan_workspace_size,
    ssm_ssd_fwd,
    ssm_ssd_workspace_size,
    ssm_ssd_step,
    ssm_step,
    ssm_step_ex,
)
