"""MI355X-native (gfx950) selective scan with a scalar decay per head.

``ssd_forward`` runs the block algorithm over whole sequences and ``ssm_step``
one decode step, both in hand-written HIP kernels behind the C ABI of
``include/ssd_mi355x.h`` (``libssd_mi355x.so``).  This package only marshals
torch tensors into that ABI.
"""
from .ssd import (  # noqa: F401
    DTYPE_BF16,
    DTYPE_F32,
    ABI_VERSION,
    SSDError,
    abi_version,
    chunk_cumsum,
    chunk_cumsum_state,
    chunk_scan,
    chunk_state,
    layer_in,
    layer_out,
    library_path,
    load,
    n_chunks,
    chunk_scan_runs,
    chunk_state_runs,
    forward_run_chunks,
    run_passing,
    ssd_forward,
    ssd_layer,
    ssm_step,
    state_passing,
    state_passing_seg,
    state_scan,
    status_str,
    workspace_bytes,
    workspace_regions,
)

__all__ = [
    "ssd_forward", "ssm_step", "workspace_bytes", "workspace_regions", "chunk_cumsum",
    "chunk_cumsum_state", "chunk_state", "state_passing", "state_scan", "chunk_scan", "load", "library_path", "abi_version",
    "status_str", "SSDError", "n_chunks", "DTYPE_F32", "DTYPE_BF16", "ABI_VERSION", "layer_in",
    "layer_out", "ssd_layer", "state_passing_seg", "chunk_state_runs", "run_passing",
    "chunk_scan_runs", "forward_run_chunks",
]
