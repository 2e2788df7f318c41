"""Linear-memory relation-KL (LinearARD) for AMD MI355X (gfx950).

Public Python surface: thin ctypes wrappers over liblarard.so.
"""
from .binding import (  # noqa: F401
    BF16, FP32, DX_AUTO, DX_SPLIT, DX_ATOMIC, DX_FUSED, LarardError, LIB_PATH, default_scale, kl_bwd, kl_fwd,
    kl_bwd_cols, kl_bwd_rows, reduce_loss,
    load, loss, loss_head_group, loss_sweep_group, lse_fwd, source_id, stat_dtype, version, workspace_bytes, workspace_layout,
    xy_kl_bwd, xy_kl_fwd, xy_loss, xy_lse_fwd, LarardMap, multi_loss, multi_workspace_bytes, proj_bwd,
    loss_noalloc, NOALLOC_SCRATCH_BYTES,
)
