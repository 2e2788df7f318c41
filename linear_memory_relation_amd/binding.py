"""ctypes binding of liblarard.so: argument marshalling only.

Every step of the relation-KL path runs in the HIP kernels behind the C ABI
(include/larard.h).  PyTorch supplies device memory and the current stream.
There is no fallback: if the library is missing or a call fails, an
exception is raised.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Tuple

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "liblarard.so")

OK, E_INVALID, E_UNSUPPORTED, E_WORKSPACE, E_HIP = 0, 1, 2, 3, 4
BF16, FP32 = 0, 1
DX_AUTO, DX_SPLIT, DX_ATOMIC, DX_FUSED = 0, 1, 2, 3

_lib: Optional[ctypes.CDLL] = None


class LarardError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        self.status = status
        super().__init__(f"{where}: {detail}")


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load liblarard.so (built by linear_memory_relation_amd.build); raises if absent."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"liblarard.so not found at {path}; build it with "
                           "`python -c 'import __graft_entry__ as g; g.build()'`")
    lib = ctypes.CDLL(path)
    vp, i64, f32, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_float, ctypes.c_int
    lib.larard_workspace_bytes.argtypes = [i32, i64, i64, i64]
    lib.larard_workspace_bytes.restype = ctypes.c_size_t
    lib.larard_loss_head_group.argtypes = [i32, i64, i64, i64, i64, i32]
    lib.larard_loss_head_group.restype = i64
    lib.larard_loss_sweep_group.argtypes = [i32, i64, i64, i64, i64, i32]
    lib.larard_loss_sweep_group.restype = i64
    lib.larard_workspace_layout.argtypes = [i32, i64, i64, i64, ctypes.POINTER(ctypes.c_size_t)]
    lib.larard_workspace_layout.restype = i32
    lib.larard_lse_fwd.argtypes = [vp, vp, i32, i64, i64, i64, i64, f32, i32, vp, vp, vp]
    lib.larard_lse_fwd.restype = i32
    lib.larard_kl_fwd.argtypes = [vp, vp, i32, i64, i64, i64, i64, f32, i32, vp, vp, vp, vp]
    lib.larard_kl_fwd.restype = i32
    lib.larard_kl_bwd.argtypes = [vp, vp, i32, i64, i64, i64, i64, f32, i32, vp, vp, f32, vp, vp, i32, vp]
    lib.larard_kl_bwd.restype = i32
    lib.larard_kl_bwd_rows.argtypes = [vp, vp, i32, i64, i64, i64, i64, f32, i32, vp, vp, f32, vp, vp, vp]
    lib.larard_kl_bwd_rows.restype = i32
    lib.larard_kl_bwd_cols.argtypes = [vp, vp, i32, i64, i64, i64, i64, f32, i32, vp, vp, f32, vp, vp]
    lib.larard_kl_bwd_cols.restype = i32
    lib.larard_reduce_loss.argtypes = [vp, i64, i64, i64, f32, vp, vp, vp]
    lib.larard_reduce_loss.restype = i32
    lib.larard_loss.argtypes = [vp, vp, i32, i64, i64, i64, i64, f32, i32, f32, vp, ctypes.c_size_t,
                                vp, vp, i32, vp]
    lib.larard_loss.restype = i32
    lib.larard_loss_noalloc.argtypes = [vp, vp, i32, i64, i64, i64, i64, f32, i32, f32, vp, vp, i32, vp]
    lib.larard_loss_noalloc.restype = i32
    lib.larard_xy_lse_fwd.argtypes = [vp, vp, vp, vp, i32, i64, i64, i64, i64, f32, i32, vp, vp, vp]
    lib.larard_xy_lse_fwd.restype = i32
    lib.larard_xy_kl_fwd.argtypes = [vp, vp, vp, vp, i32, i64, i64, i64, i64, f32, i32, vp, vp, vp, vp]
    lib.larard_xy_kl_fwd.restype = i32
    lib.larard_xy_kl_bwd.argtypes = [vp, vp, vp, vp, i32, i64, i64, i64, i64, f32, i32, vp, vp, f32, vp, vp, vp, vp]
    lib.larard_xy_kl_bwd.restype = i32
    lib.larard_xy_loss.argtypes = [vp, vp, vp, vp, i32, i64, i64, i64, i64, f32, i32, f32, vp, ctypes.c_size_t,
                                   vp, vp, vp, vp]
    lib.larard_xy_loss.restype = i32
    lib.larard_multi_workspace_bytes.argtypes = [i32, i64, i64, ctypes.POINTER(LarardMap), i32]
    lib.larard_multi_workspace_bytes.restype = ctypes.c_size_t
    lib.larard_multi_loss.argtypes = [ctypes.POINTER(LarardMap), i32, i32, i64, i64, i64, f32, i32, f32, vp,
                                      ctypes.c_size_t, vp, vp]
    lib.larard_multi_loss.restype = i32
    lib.larard_proj_bwd_workspace_bytes.argtypes = [i64, i64, i64, i64, i64]
    lib.larard_proj_bwd_workspace_bytes.restype = ctypes.c_size_t
    lib.larard_proj_bwd.argtypes = [vp, vp, i64, i64, i64, i64, i64, vp, vp, vp, ctypes.c_size_t, vp, vp]
    lib.larard_proj_bwd.restype = i32
    lib.larard_status_str.argtypes = [i32]
    lib.larard_status_str.restype = ctypes.c_char_p
    lib.larard_last_error.argtypes = []
    lib.larard_last_error.restype = ctypes.c_char_p
    lib.larard_version.argtypes = []
    lib.larard_version.restype = ctypes.c_char_p
    _lib = lib
    return lib


class LarardMap(ctypes.Structure):
    """larard_map of larard.h: one self-relation map of a multi-map launch."""
    _fields_ = [("x_t", ctypes.c_void_p), ("x_s", ctypes.c_void_p), ("H", ctypes.c_int64),
                ("weight", ctypes.c_float), ("dx_s", ctypes.c_void_p)]


def _check(status: int, where: str) -> None:
    if status != OK:
        lib = load()
        raise LarardError(status, where, f"{lib.larard_status_str(status).decode()} -- "
                                         f"{lib.larard_last_error().decode()}")


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return FP32
    raise TypeError(f"unsupported dtype {t.dtype}; use bfloat16 or float32")


def _shape(xt: torch.Tensor, xs: torch.Tensor):
    """(B, H, n, d) of a teacher/student pair; shape, dtype and layout only (the device is
    checked by _on_gpu once every buffer of the call has been checked)."""
    if not (isinstance(xt, torch.Tensor) and isinstance(xs, torch.Tensor)):
        raise ValueError("x_t and x_s must be torch tensors")
    if xt.dim() != 4 or xt.shape != xs.shape or xt.dtype != xs.dtype:
        raise ValueError("x_t and x_s must both be [B, H, n, d] with the same dtype")
    _dtype_code(xt)
    if not (xt.is_contiguous() and xs.is_contiguous()):
        raise ValueError("x_t and x_s must be contiguous")
    return tuple(int(v) for v in xt.shape)


def _need(t: Optional[torch.Tensor], name: str, shape, dtype: torch.dtype, optional: bool = False) -> None:
    """A caller-supplied buffer must be a contiguous tensor of exactly this shape and dtype
    (the kernels index it by the shape of the inputs, so anything else reads or writes out of
    bounds)."""
    if t is None:
        if optional:
            return
        raise ValueError(f"{name} is required")
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch tensor")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _need_bytes(t: Optional[torch.Tensor], name: str, nbytes: int) -> None:
    """A caller-supplied workspace: any contiguous tensor of at least nbytes bytes."""
    if t is None:
        return
    if not isinstance(t, torch.Tensor) or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous tensor")
    if t.numel() * t.element_size() < nbytes:
        raise ValueError(f"{name} must hold at least {nbytes} bytes, got {t.numel() * t.element_size()}")


def _on_gpu(*tensors: Optional[torch.Tensor]) -> None:
    """Every tensor of one call must live on the same GPU."""
    ts = [t for t in tensors if t is not None]
    if not all(t.is_cuda for t in ts):
        raise ValueError("every tensor of the call must be a GPU tensor")
    if len({t.device for t in ts}) > 1:
        raise ValueError("every tensor of the call must be on the same GPU")


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def default_scale(d: int) -> float:
    return 1.0 / math.sqrt(d)


def workspace_bytes(B: int, H: int, n: int, dtype: int = BF16) -> int:
    return int(load().larard_workspace_bytes(dtype, B, H, n))


def loss_head_group(B: int, H: int, n: int, d: int, dtype: int = BF16, cross: bool = False) -> int:
    """Heads per group of the whole-path calls (phase 1 and 2 per group of the B*H heads)."""
    g = int(load().larard_loss_head_group(dtype, B, H, n, d, 1 if cross else 0))
    if g <= 0:
        raise ValueError(f"invalid sizes B={B} H={H} n={n} d={d}")
    return g


def loss_sweep_group(B: int, H: int, n: int, d: int, dtype: int = BF16, cross: bool = False) -> int:
    """Heads per phase-2 sub-group of the whole-path calls (within each head group)."""
    g = int(load().larard_loss_sweep_group(dtype, B, H, n, d, 1 if cross else 0))
    if g <= 0:
        raise ValueError(f"invalid sizes B={B} H={H} n={n} d={d}")
    return g


def workspace_layout(B: int, H: int, n: int, dtype: int = BF16):
    off = (ctypes.c_size_t * 4)()
    _check(load().larard_workspace_layout(dtype, B, H, n, off), "larard_workspace_layout")
    return [int(v) for v in off]


def stat_dtype(x: torch.Tensor) -> torch.dtype:
    """Element type of the LSE statistics (fp64 for every input type)."""
    return torch.float64


def lse_fwd(xt: torch.Tensor, xs: torch.Tensor, scale: Optional[float] = None, causal: bool = True,
            lse_t: Optional[torch.Tensor] = None, lse_s: Optional[torch.Tensor] = None
            ) -> Tuple[torch.Tensor, torch.Tensor]:
    """Phase 1: per-row log-sum-exp of teacher and student logits, fp64 [B, H, n]."""
    B, H, n, d = _shape(xt, xs)
    scale = default_scale(d) if scale is None else float(scale)
    _need(lse_t, "lse_t", (B, H, n), torch.float64, optional=True)
    _need(lse_s, "lse_s", (B, H, n), torch.float64, optional=True)
    _on_gpu(xt, xs, lse_t, lse_s)
    if lse_t is None:
        lse_t = torch.empty((B, H, n), dtype=stat_dtype(xt), device=xt.device)
    if lse_s is None:
        lse_s = torch.empty((B, H, n), dtype=stat_dtype(xt), device=xt.device)
    st = load().larard_lse_fwd(_ptr(xt), _ptr(xs), _dtype_code(xt), B, H, n, d, scale, int(causal),
                               _ptr(lse_t), _ptr(lse_s), _stream())
    _check(st, "larard_lse_fwd")
    return lse_t, lse_s


def kl_fwd(xt: torch.Tensor, xs: torch.Tensor, scale: Optional[float] = None, causal: bool = True,
           lse_t: Optional[torch.Tensor] = None, lse_s: Optional[torch.Tensor] = None,
           row_kl: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """Forward-only sweep: (lse_t, lse_s, row_kl) -- fp64, fp64, fp32 [B, H, n] -- in one pass."""
    B, H, n, d = _shape(xt, xs)
    scale = default_scale(d) if scale is None else float(scale)
    _need(lse_t, "lse_t", (B, H, n), torch.float64, optional=True)
    _need(lse_s, "lse_s", (B, H, n), torch.float64, optional=True)
    _need(row_kl, "row_kl", (B, H, n), torch.float32, optional=True)
    _on_gpu(xt, xs, lse_t, lse_s, row_kl)
    if lse_t is None:
        lse_t = torch.empty((B, H, n), dtype=stat_dtype(xt), device=xt.device)
    if lse_s is None:
        lse_s = torch.empty((B, H, n), dtype=stat_dtype(xt), device=xt.device)
    if row_kl is None:
        row_kl = torch.empty((B, H, n), dtype=torch.float32, device=xt.device)
    st = load().larard_kl_fwd(_ptr(xt), _ptr(xs), _dtype_code(xt), B, H, n, d, scale, int(causal),
                              _ptr(lse_t), _ptr(lse_s), _ptr(row_kl), _stream())
    _check(st, "larard_kl_fwd")
    return lse_t, lse_s, row_kl


def kl_bwd(xt: torch.Tensor, xs: torch.Tensor, lse_t: torch.Tensor, lse_s: torch.Tensor,
           scale: Optional[float] = None, causal: bool = True, loss_scale: float = 1.0,
           need_dx: bool = True, dx_mode: int = DX_AUTO, row_kl: Optional[torch.Tensor] = None,
           dx: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Phase 2: per-row KL(R_t || R_s) (fp32 [B,H,n]) and dX_s (fp32 [B,H,n,d] or None)."""
    B, H, n, d = _shape(xt, xs)
    scale = default_scale(d) if scale is None else float(scale)
    if not need_dx:
        dx = None
    _need(lse_t, "lse_t", (B, H, n), torch.float64)
    _need(lse_s, "lse_s", (B, H, n), torch.float64)
    _need(row_kl, "row_kl", (B, H, n), torch.float32, optional=True)
    _need(dx, "dx", (B, H, n, d), torch.float32, optional=True)
    _on_gpu(xt, xs, lse_t, lse_s, row_kl, dx)
    if row_kl is None:
        row_kl = torch.empty((B, H, n), dtype=torch.float32, device=xt.device)
    if need_dx and dx is None:
        dx = torch.empty((B, H, n, d), dtype=torch.float32, device=xt.device)
    st = load().larard_kl_bwd(_ptr(xt), _ptr(xs), _dtype_code(xt), B, H, n, d, scale, int(causal),
                              _ptr(lse_t), _ptr(lse_s), float(loss_scale), _ptr(row_kl), _ptr(dx),
                              int(dx_mode), _stream())
    _check(st, "larard_kl_bwd")
    return row_kl, dx


def kl_bwd_rows(xt, xs, lse_t, lse_s, row_kl, dx=None, scale=None, causal=True, loss_scale=1.0):
    """Row-owned half of phase 2: writes row_kl, stores the row term into dx (if given)."""
    B, H, n, d = _shape(xt, xs)
    scale = default_scale(d) if scale is None else float(scale)
    _need(lse_t, "lse_t", (B, H, n), torch.float64)
    _need(lse_s, "lse_s", (B, H, n), torch.float64)
    _need(row_kl, "row_kl", (B, H, n), torch.float32)
    _need(dx, "dx", (B, H, n, d), torch.float32, optional=True)
    _on_gpu(xt, xs, lse_t, lse_s, row_kl, dx)
    st = load().larard_kl_bwd_rows(_ptr(xt), _ptr(xs), _dtype_code(xt), B, H, n, d, scale, int(causal),
                                   _ptr(lse_t), _ptr(lse_s), float(loss_scale), _ptr(row_kl), _ptr(dx),
                                   _stream())
    _check(st, "larard_kl_bwd_rows")


def kl_bwd_cols(xt, xs, lse_t, lse_s, dx, scale=None, causal=True, loss_scale=1.0):
    """Column-owned half of phase 2: adds the column term into dx."""
    B, H, n, d = _shape(xt, xs)
    scale = default_scale(d) if scale is None else float(scale)
    _need(lse_t, "lse_t", (B, H, n), torch.float64)
    _need(lse_s, "lse_s", (B, H, n), torch.float64)
    _need(dx, "dx", (B, H, n, d), torch.float32)
    _on_gpu(xt, xs, lse_t, lse_s, dx)
    st = load().larard_kl_bwd_cols(_ptr(xt), _ptr(xs), _dtype_code(xt), B, H, n, d, scale, int(causal),
                                   _ptr(lse_t), _ptr(lse_s), float(loss_scale), _ptr(dx), _stream())
    _check(st, "larard_kl_bwd_cols")


def reduce_loss(row_kl: torch.Tensor, partials: torch.Tensor, out: torch.Tensor, loss_scale: float = 1.0):
    """loss = loss_scale * sum over heads of the row mean of row_kl ([B, H, n] fp32)."""
    if not isinstance(row_kl, torch.Tensor) or row_kl.dim() != 3:
        raise ValueError("row_kl must be a [B, H, n] tensor")
    B, H, n = (int(v) for v in row_kl.shape)
    _need(row_kl, "row_kl", (B, H, n), torch.float32)
    _need(partials, "partials", (B * H,), torch.float64)
    _need(out, "out", (), torch.float32)
    _on_gpu(row_kl, partials, out)
    st = load().larard_reduce_loss(_ptr(row_kl), B, H, n, float(loss_scale), _ptr(partials), _ptr(out),
                                   _stream())
    _check(st, "larard_reduce_loss")


def loss(xt: torch.Tensor, xs: torch.Tensor, scale: Optional[float] = None, causal: bool = True,
         loss_scale: float = 1.0, need_dx: bool = True, dx_mode: int = DX_AUTO,
         workspace: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
         dx: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Whole path for one relation map: returns (loss as a 0-d fp32 device tensor, dX_s or None)."""
    B, H, n, d = _shape(xt, xs)
    scale = default_scale(d) if scale is None else float(scale)
    nbytes = workspace_bytes(B, H, n, _dtype_code(xt))
    if not need_dx:
        dx = None
    _need_bytes(workspace, "workspace", nbytes)
    _need(out, "out", (), torch.float32, optional=True)
    _need(dx, "dx", (B, H, n, d), torch.float32, optional=True)
    _on_gpu(xt, xs, workspace, out, dx)
    if workspace is None:
        workspace = torch.empty((max(nbytes, 256),), dtype=torch.uint8, device=xt.device)
    if out is None:
        out = torch.empty((), dtype=torch.float32, device=xt.device)
    if need_dx and dx is None:
        dx = torch.empty((B, H, n, d), dtype=torch.float32, device=xt.device)
    st = load().larard_loss(_ptr(xt), _ptr(xs), _dtype_code(xt), B, H, n, d, scale, int(causal),
                            float(loss_scale), _ptr(workspace), workspace.numel() * workspace.element_size(),
                            _ptr(out), _ptr(dx), int(dx_mode), _stream())
    _check(st, "larard_loss")
    return out, dx


NOALLOC_SCRATCH_BYTES = 64 << 20      # LARARD_NOALLOC_SCRATCH_BYTES of larard.h


def loss_noalloc(xt: torch.Tensor, xs: torch.Tensor, scale: Optional[float] = None, causal: bool = True,
                 loss_scale: float = 1.0, need_dx: bool = True, dx_mode: int = DX_AUTO,
                 out: Optional[torch.Tensor] = None, dx: Optional[torch.Tensor] = None
                 ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """larard_loss_noalloc: the whole path for one map with the library's static device scratch
    (no workspace; the caller's out/dx are the only buffers).  Same results as `loss`."""
    B, H, n, d = _shape(xt, xs)
    scale = default_scale(d) if scale is None else float(scale)
    if not need_dx:
        dx = None
    _need(out, "out", (), torch.float32, optional=True)
    _need(dx, "dx", (B, H, n, d), torch.float32, optional=True)
    _on_gpu(xt, xs, out, dx)
    if out is None:
        out = torch.empty((), dtype=torch.float32, device=xt.device)
    if need_dx and dx is None:
        dx = torch.empty((B, H, n, d), dtype=torch.float32, device=xt.device)
    st = load().larard_loss_noalloc(_ptr(xt), _ptr(xs), _dtype_code(xt), B, H, n, d, scale, int(causal),
                                    float(loss_scale), _ptr(out), _ptr(dx), int(dx_mode), _stream())
    _check(st, "larard_loss_noalloc")
    return out, dx


# ---------------------------------------------------------------------------
# General relation X != Y: Z = scale * X Y^T, gradients dX_s and dY_s.
# ---------------------------------------------------------------------------
def _shape_xy(xt, xs, yt, ys):
    shp = _shape(xt, xs)
    if _shape(yt, ys) != shp or yt.dtype != xt.dtype:
        raise ValueError("y_t, y_s must match x_t, x_s in shape and dtype")
    return shp


def _xy_stats(B, H, n, lse_t, lse_s, row_kl, required: bool):
    _need(lse_t, "lse_t", (B, H, n), torch.float64, optional=not required)
    _need(lse_s, "lse_s", (B, H, n), torch.float64, optional=not required)
    _need(row_kl, "row_kl", (B, H, n), torch.float32, optional=True)


def xy_lse_fwd(xt, xs, yt, ys, scale=None, causal=True, lse_t=None, lse_s=None):
    """Phase 1 of the X/Y relation: (lse_t, lse_s), fp64 [B, H, n]."""
    B, H, n, d = _shape_xy(xt, xs, yt, ys)
    scale = default_scale(d) if scale is None else float(scale)
    _xy_stats(B, H, n, lse_t, lse_s, None, False)
    _on_gpu(xt, xs, yt, ys, lse_t, lse_s)
    lse_t = torch.empty((B, H, n), dtype=torch.float64, device=xt.device) if lse_t is None else lse_t
    lse_s = torch.empty((B, H, n), dtype=torch.float64, device=xt.device) if lse_s is None else lse_s
    st = load().larard_xy_lse_fwd(_ptr(xt), _ptr(xs), _ptr(yt), _ptr(ys), _dtype_code(xt), B, H, n, d, scale,
                                  int(causal), _ptr(lse_t), _ptr(lse_s), _stream())
    _check(st, "larard_xy_lse_fwd")
    return lse_t, lse_s


def xy_kl_fwd(xt, xs, yt, ys, scale=None, causal=True, lse_t=None, lse_s=None, row_kl=None):
    """Forward-only X/Y relation in one sweep: (lse_t, lse_s, row_kl)."""
    B, H, n, d = _shape_xy(xt, xs, yt, ys)
    scale = default_scale(d) if scale is None else float(scale)
    _xy_stats(B, H, n, lse_t, lse_s, row_kl, False)
    _on_gpu(xt, xs, yt, ys, lse_t, lse_s, row_kl)
    lse_t = torch.empty((B, H, n), dtype=torch.float64, device=xt.device) if lse_t is None else lse_t
    lse_s = torch.empty((B, H, n), dtype=torch.float64, device=xt.device) if lse_s is None else lse_s
    row_kl = torch.empty((B, H, n), dtype=torch.float32, device=xt.device) if row_kl is None else row_kl
    st = load().larard_xy_kl_fwd(_ptr(xt), _ptr(xs), _ptr(yt), _ptr(ys), _dtype_code(xt), B, H, n, d, scale,
                                 int(causal), _ptr(lse_t), _ptr(lse_s), _ptr(row_kl), _stream())
    _check(st, "larard_xy_kl_fwd")
    return lse_t, lse_s, row_kl


def xy_kl_bwd(xt, xs, yt, ys, lse_t, lse_s, scale=None, causal=True, loss_scale=1.0, need_dx=True,
              need_dy=True, row_kl=None, dx=None, dy=None):
    """Phase 2 of the X/Y relation: (row_kl, dX_s or None, dY_s or None)."""
    B, H, n, d = _shape_xy(xt, xs, yt, ys)
    scale = default_scale(d) if scale is None else float(scale)
    dx = dx if need_dx else None
    dy = dy if need_dy else None
    _xy_stats(B, H, n, lse_t, lse_s, row_kl, True)
    _need(dx, "dx", (B, H, n, d), torch.float32, optional=True)
    _need(dy, "dy", (B, H, n, d), torch.float32, optional=True)
    _on_gpu(xt, xs, yt, ys, lse_t, lse_s, row_kl, dx, dy)
    row_kl = torch.empty((B, H, n), dtype=torch.float32, device=xt.device) if row_kl is None else row_kl
    dx = (torch.empty((B, H, n, d), dtype=torch.float32, device=xt.device) if dx is None else dx) if need_dx else None
    dy = (torch.empty((B, H, n, d), dtype=torch.float32, device=xt.device) if dy is None else dy) if need_dy else None
    st = load().larard_xy_kl_bwd(_ptr(xt), _ptr(xs), _ptr(yt), _ptr(ys), _dtype_code(xt), B, H, n, d, scale,
                                 int(causal), _ptr(lse_t), _ptr(lse_s), float(loss_scale), _ptr(row_kl),
                                 _ptr(dx), _ptr(dy), _stream())
    _check(st, "larard_xy_kl_bwd")
    return row_kl, dx, dy


def xy_loss(xt, xs, yt, ys, scale=None, causal=True, loss_scale=1.0, need_grad=True, workspace=None,
            out=None, dx=None, dy=None):
    """Whole X/Y path for one relation map: (loss 0-d fp32 tensor, dX_s or None, dY_s or None)."""
    B, H, n, d = _shape_xy(xt, xs, yt, ys)
    scale = default_scale(d) if scale is None else float(scale)
    nbytes = workspace_bytes(B, H, n, _dtype_code(xt))
    if not need_grad:
        dx = dy = None
    _need_bytes(workspace, "workspace", nbytes)
    _need(out, "out", (), torch.float32, optional=True)
    _need(dx, "dx", (B, H, n, d), torch.float32, optional=True)
    _need(dy, "dy", (B, H, n, d), torch.float32, optional=True)
    _on_gpu(xt, xs, yt, ys, workspace, out, dx, dy)
    if workspace is None:
        workspace = torch.empty((max(nbytes, 256),), dtype=torch.uint8, device=xt.device)
    out = torch.empty((), dtype=torch.float32, device=xt.device) if out is None else out
    if need_grad:
        dx = torch.empty((B, H, n, d), dtype=torch.float32, device=xt.device) if dx is None else dx
        dy = torch.empty((B, H, n, d), dtype=torch.float32, device=xt.device) if dy is None else dy
    else:
        dx = dy = None
    st = load().larard_xy_loss(_ptr(xt), _ptr(xs), _ptr(yt), _ptr(ys), _dtype_code(xt), B, H, n, d, scale,
                               int(causal), float(loss_scale), _ptr(workspace),
                               workspace.numel() * workspace.element_size(), _ptr(out), _ptr(dx), _ptr(dy),
                               _stream())
    _check(st, "larard_xy_loss")
    return out, dx, dy


# ---------------------------------------------------------------------------
# Several self-relation maps (e.g. Q/Q, K/K, V/V with GQA head counts) in one
# launch per phase.
# ---------------------------------------------------------------------------
def _map_array(maps):
    arr = (LarardMap * len(maps))()
    for k, (xt, xs, weight, dx) in enumerate(maps):
        arr[k] = LarardMap(_ptr(xt), _ptr(xs), int(xt.shape[1]), float(weight), _ptr(dx))
    return arr


def multi_workspace_bytes(maps, dtype: int = BF16) -> int:
    """maps: list of (x_t, x_s, weight, dx or None) with x [B, H_m, n, d]."""
    B, _, n, _ = (int(v) for v in maps[0][0].shape)
    return int(load().larard_multi_workspace_bytes(dtype, B, n, _map_array(maps), len(maps)))


def multi_loss(maps, scale: Optional[float] = None, causal: bool = True, loss_scale: float = 1.0,
               workspace: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Weighted loss over several maps in one launch per phase.

    maps: list of (x_t, x_s, weight, dx) -- dx an fp32 [B, H_m, n, d] tensor that
    receives that map's gradient, or None for every map (loss only).
    Returns the loss as a 0-d fp32 device tensor.
    """
    if not maps:
        raise ValueError("maps must not be empty")
    xt0 = maps[0][0]
    _shape(xt0, maps[0][1])
    B, _, n, d = (int(v) for v in xt0.shape)
    for k, (xt, xs, _, dx) in enumerate(maps):
        _, Hm, _, _ = _shape(xt, xs)
        if xt.shape[0] != B or xt.shape[2] != n or xt.shape[3] != d or xt.dtype != xt0.dtype:
            raise ValueError("maps must share B, n, d and dtype")
        _need(dx, f"dx of map {k}", (B, Hm, n, d), torch.float32, optional=True)
    scale = default_scale(d) if scale is None else float(scale)
    arr = _map_array(maps)
    code = _dtype_code(xt0)
    nbytes = int(load().larard_multi_workspace_bytes(code, B, n, arr, len(maps)))
    _need_bytes(workspace, "workspace", nbytes)
    _need(out, "out", (), torch.float32, optional=True)
    _on_gpu(*[t for xt, xs, _, dx in maps for t in (xt, xs, dx)], workspace, out)
    if workspace is None:
        workspace = torch.empty((max(nbytes, 256),), dtype=torch.uint8, device=xt0.device)
    out = torch.empty((), dtype=torch.float32, device=xt0.device) if out is None else out
    st = load().larard_multi_loss(arr, len(maps), code, B, n, d, scale, int(causal), float(loss_scale),
                                  _ptr(workspace), workspace.numel() * workspace.element_size(), _ptr(out),
                                  _stream())
    _check(st, "larard_multi_loss")
    return out


# ---------------------------------------------------------------------------
# Projection backward: dW = h^T R^T(dX_s).
# ---------------------------------------------------------------------------
def proj_bwd(h: torch.Tensor, dx_s: torch.Tensor, rope_cos: Optional[torch.Tensor] = None,
             rope_sin: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
             out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """h: bf16 [B, n, dm]; dx_s: fp32 [B, H, n, d]; rope tables fp32 [n, d/2] or None.
    Returns dW fp32 [dm, H*d]."""
    if not (isinstance(h, torch.Tensor) and isinstance(dx_s, torch.Tensor)) or h.dim() != 3 or dx_s.dim() != 4:
        raise ValueError("h must be bf16 [B, n, dm] and dx_s fp32 [B, H, n, d]")
    B, n, dm = (int(v) for v in h.shape)
    _, H, n2, d = (int(v) for v in dx_s.shape)
    if n2 != n or dx_s.shape[0] != B or h.dtype != torch.bfloat16 or dx_s.dtype != torch.float32:
        raise ValueError("h must be bf16 [B, n, dm] and dx_s fp32 [B, H, n, d]")
    if not (h.is_contiguous() and dx_s.is_contiguous()):
        raise ValueError("h and dx_s must be contiguous")
    if (rope_cos is None) != (rope_sin is None):
        raise ValueError("rope_cos and rope_sin must both be given or both be None")
    # Half-width tables: entry [i, k] turns the pair (k, k + d/2) of token i.
    _need(rope_cos, "rope_cos", (n, d // 2), torch.float32, optional=True)
    _need(rope_sin, "rope_sin", (n, d // 2), torch.float32, optional=True)
    _need(out, "out", (dm, H * d), torch.float32, optional=True)
    nbytes = int(load().larard_proj_bwd_workspace_bytes(B, n, dm, H, d))
    _need_bytes(workspace, "workspace", nbytes)
    _on_gpu(h, dx_s, rope_cos, rope_sin, workspace, out)
    if workspace is None:
        workspace = torch.empty((max(nbytes, 256),), dtype=torch.uint8, device=h.device)
    out = torch.empty((dm, H * d), dtype=torch.float32, device=h.device) if out is None else out
    st = load().larard_proj_bwd(_ptr(h), _ptr(dx_s), B, n, dm, H, d, _ptr(rope_cos), _ptr(rope_sin),
                                _ptr(workspace), workspace.numel() * workspace.element_size(), _ptr(out),
                                _stream())
    _check(st, "larard_proj_bwd")
    return out


def version() -> str:
    return load().larard_version().decode()


def source_id() -> str:
    """Hash of the sources the loaded library was built from (from its version string)."""
    v = version()
    return v.split("(src ", 1)[1].rstrip(")") if "(src " in v else ""
