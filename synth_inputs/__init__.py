"""Seeded synthetic teacher/student projections for the relation-KL path.

This module only *prepares inputs*: it draws seeded Gaussian projections,
applies rotary position embeddings (RoPE) at teacher and student positions or
bases, and rounds the result once to the storage precision.  It contains none
of the relation-KL arithmetic, so both the fp64 oracle and the HIP path can
consume the same arrays without sharing any of the method's code.

Workloads stand in for the top-layer Q/K/V activations of LLaMA2-7B,
LLaMA3-8B and Mistral-7B on native-length text ("LinearARD: Linear-Memory
Attention Distillation for RoPE Restoration", notes page, section "Main
experiments" and "Loss / training strategy"); those weights and texts are not
available, so N(0,1) projections of the same shapes are used instead.

Readings (the pages print no RoPE formula):
  * RoPE uses the rotate-half pairing (k, k + d/2) with inverse frequencies
    base**(-2k/d); the teacher rotates token i by angle i*theta_k.
  * Position interpolation (PI) by a factor alpha rotates the student at
    position i/alpha; NTK-style scaling by a factor f uses the base
    base * f**(d/(d-2)) at position i.
  * V carries no RoPE; the student V is the teacher V plus N(0, 0.05^2) noise.
  * RoPE and noise are applied in float64 and the result is rounded once
    (round-to-nearest-even) to bf16 or fp32.
"""
from __future__ import annotations

import concurrent.futures as _cf
import dataclasses
import math
import os
from typing import Dict, List, Optional

import numpy as np

__all__ = [
    "Workload", "MapInputs", "WORKLOADS", "workload", "make_inputs",
    "rope_tables", "apply_rope", "round_bf16_bits", "bf16_bits_to_f64",
    "round_f32",
]


# --------------------------------------------------------------------------
# Rounding helpers
# --------------------------------------------------------------------------

def round_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float64 values once, to nearest-even, to bf16; return uint16 bits.

    bf16 keeps 1 sign, 8 exponent and 7 mantissa bits (the top half of an
    IEEE binary32).  The rounding is done on the binary64 bit pattern (52 ->
    7 mantissa bits), so there is exactly one rounding step.  Inputs must be
    finite and inside the normal bf16 range (true for these workloads).
    """
    x = np.ascontiguousarray(x, dtype=np.float64)
    bits = x.view(np.uint64)
    drop = np.uint64(45)                       # 52 - 7 mantissa bits dropped
    lsb = (bits >> drop) & np.uint64(1)
    half = np.uint64((1 << 44) - 1)
    rounded = ((bits + half + lsb) >> drop) << drop
    y = rounded.view(np.float64).astype(np.float32)   # exact: 8-bit significand
    return (y.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact float64 image of bf16 bit patterns."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def round_f32(x: np.ndarray) -> np.ndarray:
    """Round float64 once to float32 (numpy casts round to nearest-even)."""
    return np.asarray(x, dtype=np.float64).astype(np.float32)


# --------------------------------------------------------------------------
# RoPE (input preparation only)
# --------------------------------------------------------------------------

def rope_tables(n: int, d: int, base: float, pos_scale: float = 1.0):
    """cos/sin tables [n, d] (float64) for rotate-half RoPE.

    Token i is rotated at position i / pos_scale; pair k (and k + d/2) uses the
    inverse frequency base**(-2k/d).
    """
    k = np.arange(d // 2, dtype=np.float64)
    inv_freq = base ** (-2.0 * k / d)
    pos = np.arange(n, dtype=np.float64) / pos_scale
    ang = np.outer(pos, inv_freq)
    ang = np.concatenate([ang, ang], axis=1)
    return np.cos(ang), np.sin(ang)


def apply_rope(x: np.ndarray, cos: np.ndarray, sin: np.ndarray) -> np.ndarray:
    """Rotate-half RoPE in float64: x*cos + rotate_half(x)*sin, over [..., n, d]."""
    x = np.asarray(x, dtype=np.float64)
    h = x.shape[-1] // 2
    rot = np.concatenate([-x[..., h:], x[..., :h]], axis=-1)
    return x * cos + rot * sin


# --------------------------------------------------------------------------
# Workloads
# --------------------------------------------------------------------------

@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    n: int
    d: int
    dtype: str                     # "bf16" or "f32"
    heads: Dict[str, int]          # map name -> head count
    seed: int
    kind: str                      # "pi" or "ntk"
    base: float                    # teacher RoPE base
    factor: float                  # PI alpha or NTK factor
    per_head_scale: bool = False   # Q/K projections scaled by U(0.5, 2) per head
    v_noise: float = 0.05

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    def head_maps(self) -> int:
        return sum(self.B * h for h in self.heads.values())


WORKLOADS: Dict[str, Workload] = {
    # Tiny fp32 Q/Q relation (n=256, d=64, PI x4).
    "tiny_f32": Workload("tiny_f32", 1, 256, 64, "f32", {"Q": 1}, 0,
                         "pi", 1.0e4, 4.0),
    # LLaMA2-7B top-layer heads at native length 4K, PI x8, Q/Q+K/K+V/V.
    "llama2_4k": Workload("llama2_4k", 1, 4096, 128, "bf16",
                          {"Q": 32, "K": 32, "V": 32}, 1, "pi", 1.0e4, 8.0),
    # Same construction at n=16K (length where the dense n x n map no longer
    # fits a 96 GB card).
    "llama2_16k": Workload("llama2_16k", 1, 16384, 128, "bf16",
                           {"Q": 32, "K": 32, "V": 32}, 2, "pi", 1.0e4, 8.0),
    # Same construction at n=32K (4K -> 32K extension length).
    "llama2_32k": Workload("llama2_32k", 1, 32768, 128, "bf16",
                           {"Q": 32, "K": 32, "V": 32}, 3, "pi", 1.0e4, 8.0),
    # LLaMA3-8B GQA shapes: 32 Q heads, 8 KV heads, B=2, n=8K, NTK x4 student.
    "llama3_gqa_8k": Workload("llama3_gqa_8k", 2, 8192, 128, "bf16",
                              {"Q": 32, "K": 8, "V": 8}, 4, "ntk", 5.0e5, 4.0,
                              per_head_scale=True),
}


def workload(name: str, **overrides) -> Workload:
    """A named workload, optionally with fields replaced (e.g. a shorter n)."""
    return dataclasses.replace(WORKLOADS[name], **overrides)


@dataclasses.dataclass
class MapInputs:
    """One relation map's inputs. `xt`/`xs` are [B, H, n, d] storage arrays
    (uint16 bf16 bits, or float32); `xt64`/`xs64` their exact float64 images."""
    name: str
    xt: np.ndarray
    xs: np.ndarray
    dtype: str

    @property
    def xt64(self) -> np.ndarray:
        return _widen(self.xt, self.dtype)

    @property
    def xs64(self) -> np.ndarray:
        return _widen(self.xs, self.dtype)

    def head64(self, b: int, h: int):
        """Float64 images (X_t, X_s) of one head, each [n, d]."""
        return (_widen(self.xt[b, h], self.dtype), _widen(self.xs[b, h], self.dtype))


def _widen(a: np.ndarray, dtype: str) -> np.ndarray:
    return bf16_bits_to_f64(a) if dtype == "bf16" else a.astype(np.float64)


def _store(x64: np.ndarray, dtype: str) -> np.ndarray:
    return round_bf16_bits(x64) if dtype == "bf16" else round_f32(x64)


def _student_tables(w: Workload, n: int):
    if w.kind == "pi":
        return rope_tables(n, w.d, w.base, pos_scale=w.factor)
    base_s = w.base * w.factor ** (w.d / (w.d - 2))
    return rope_tables(n, w.d, base_s, pos_scale=1.0)


def _per_head(fn, B: int, H: int) -> None:
    """Run fn(b, h) for every head on a small thread pool (numpy releases the GIL)."""
    jobs = [(b, h) for b in range(B) for h in range(H)]
    workers = max(1, min(8, os.cpu_count() or 1, len(jobs)))
    if workers == 1:
        for bh in jobs:
            fn(*bh)
        return
    with _cf.ThreadPoolExecutor(max_workers=workers) as ex:
        list(ex.map(lambda bh: fn(*bh), jobs))


def _rope_pair(p32: np.ndarray, w: Workload, tabs, dtype: str):
    """Teacher and student storage arrays for projections p32 [B, H, n, d]."""
    (ct, st), (cs, ss) = tabs
    xt = np.empty(p32.shape, dtype=np.uint16 if dtype == "bf16" else np.float32)
    xs = np.empty_like(xt)

    def one(b, h):                          # per head keeps float64 temporaries small
        p = p32[b, h].astype(np.float64)
        xt[b, h] = _store(apply_rope(p, ct, st), dtype)
        xs[b, h] = _store(apply_rope(p, cs, ss), dtype)

    _per_head(one, p32.shape[0], p32.shape[1])
    return xt, xs


def make_inputs(w: Workload, maps: Optional[List[str]] = None) -> Dict[str, MapInputs]:
    """Draw every map of workload `w` (in a fixed order) and return the requested ones.

    Draw order from numpy.random.default_rng(seed): [per-head scales for Q,
    then for K/V when enabled], P_q, P_k, V_t, eps_V.  Every draw is made even
    when a map is not requested, so a map's values never depend on `maps`.
    """
    maps = list(w.heads) if maps is None else list(maps)
    rng = np.random.default_rng(w.seed)
    B, n, d = w.B, w.n, w.d
    hq = w.heads.get("Q", 0)
    hkv = w.heads.get("K", 0)
    cq = ckv = None
    if w.per_head_scale:
        cq = rng.uniform(0.5, 2.0, size=hq)
        ckv = rng.uniform(0.5, 2.0, size=hkv)
    tabs = (rope_tables(n, d, w.base, 1.0), _student_tables(w, n))
    out: Dict[str, MapInputs] = {}

    p_q = rng.standard_normal((B, hq, n, d), dtype=np.float32)
    if "Q" in maps:
        if cq is not None:
            p_q = (p_q * cq[None, :, None, None].astype(np.float32)).astype(np.float32)
        xt, xs = _rope_pair(p_q, w, tabs, w.dtype)
        out["Q"] = MapInputs("Q", xt, xs, w.dtype)
    del p_q
    if hkv == 0:
        return out
    p_k = rng.standard_normal((B, hkv, n, d), dtype=np.float32)
    if "K" in maps:
        if ckv is not None:
            p_k = (p_k * ckv[None, :, None, None].astype(np.float32)).astype(np.float32)
        xt, xs = _rope_pair(p_k, w, tabs, w.dtype)
        out["K"] = MapInputs("K", xt, xs, w.dtype)
    del p_k
    hv = w.heads.get("V", 0)
    v_t = rng.standard_normal((B, hv, n, d), dtype=np.float32)
    eps = rng.standard_normal((B, hv, n, d), dtype=np.float32)
    if "V" in maps:
        xt = np.empty(v_t.shape, dtype=np.uint16 if w.dtype == "bf16" else np.float32)
        xs = np.empty_like(xt)

        def one(b, h):
            vt = v_t[b, h].astype(np.float64)
            xt[b, h] = _store(vt, w.dtype)
            xs[b, h] = _store(vt + w.v_noise * eps[b, h].astype(np.float64), w.dtype)

        _per_head(one, B, hv)
        out["V"] = MapInputs("V", xt, xs, w.dtype)
    return out
