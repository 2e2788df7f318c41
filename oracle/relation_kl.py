"""Plain, dense, float64 oracle of the relation-KL loss and its student gradient.

TEST INFRASTRUCTURE.  Only `tests/`, the smoke check in `__graft_entry__.py`
and the CPU-baseline leg of `bench.py` may import this module.  It shares no
code, header, table or helper with the HIP library; both sides receive the
same seeded arrays from `synth_inputs`.

Source of the definitions: "LinearARD: Linear-Memory Attention Distillation
for RoPE Restoration" (paper-notes page), section "Key designs":
  item 1 (top-layer Q/K/V self-relation alignment): for teacher t and student
     s, projected sequences X_m, Y_m in R^{n x d} are causally masked and
     row-softmax normalised into a relation map R_m; (X, Y) is instantiated as
     (Q, Q), (K, K), (V, V); the loss is the sum over the three maps of the
     row-averaged forward KL divergence.  (The page's equations are lost in
     extraction; the prose above is what survives.)
  item 2 (forward-KL gradient): the forward KL's derivative w.r.t. a student
     logit stays proportional to -r_t when r_s -> 0.
  item 3 (IO-aware linear-memory operator): LSE_m(i) = log sum_k exp(Z_m(i,k))
     per row; dZ = (R_s - R_t)/n; the gradient is contracted with the
     projection vectors into dX_s and dY_s; the result is claimed to be
     exactly equal to dense full backpropagation.
The abstract page ("Abstract") repeats that KL and gradients are exact.
Because the method is claimed exact, the oracle is simply the dense
definition written out; it never tiles, fuses or reorders.

Readings where the pages are silent (each is listed with its reason in the
design notes):
  * Z_m = scale * X_m Y_m^T; `scale` is an argument (1/sqrt(d) in the
    workloads).
  * Causal mask keeps j <= i (diagonal included); masked logits are -inf and
    contribute exactly zero probability and zero KL.  causal=False keeps all
    n columns.
  * Row mean divides by n (every row, including the trivial row 0).
  * Per head the loss is (1/n) sum_i KL_i; heads are summed, and both loss and
    gradient are multiplied by `loss_scale`.
  * KL direction is KL(R_t || R_s) (teacher is the target); the teacher is
    frozen, so only student gradients are returned.
  * log R_m is formed as Z_m - LSE_m, never as log(exp(.)).
  * With Y = X (the self-relation maps), dX_s receives both contributions:
    dX_s = scale * (dZ Y_s + dZ^T X_s).
"""
from __future__ import annotations

from typing import Dict, Iterable, Optional

import numpy as np

_NEG_INF = -np.inf


def _mask(n_rows: int, n_cols: int, causal: bool, row0: int = 0) -> np.ndarray:
    """Boolean keep-mask for rows row0..row0+n_rows-1 and columns 0..n_cols-1."""
    if not causal:
        return np.ones((n_rows, n_cols), dtype=bool)
    i = np.arange(row0, row0 + n_rows)[:, None]
    j = np.arange(n_cols)[None, :]
    return j <= i


def _logsumexp_rows(z: np.ndarray) -> np.ndarray:
    """Stable row-wise log sum exp over entries that are not -inf."""
    m = np.max(z, axis=1)
    safe_m = np.where(np.isfinite(m), m, 0.0)
    return safe_m + np.log(np.sum(np.exp(z - safe_m[:, None]), axis=1))


def relation_kl_head(xt: np.ndarray, xs: np.ndarray, scale: float,
                     causal: bool = True, yt: Optional[np.ndarray] = None,
                     ys: Optional[np.ndarray] = None) -> Dict[str, np.ndarray]:
    """Dense relation KL of one head (notes page, "Key designs" items 1 and 3).

    xt, xs: [n, d] teacher / student X; yt, ys: [n, d] teacher / student Y
    (default: Y = X, the self-relation maps Q/Q, K/K, V/V).
    Returns float64 arrays: lse_t, lse_s [n]; row_kl [n]; loss (scalar, row
    mean); dz [n, n]; dxs, dys [n, d] (the two contractions of item 3); and
    dself [n, d] = dxs + dys, the total student gradient when Y = X.
    """
    xt = np.asarray(xt, dtype=np.float64)
    xs = np.asarray(xs, dtype=np.float64)
    yt = xt if yt is None else np.asarray(yt, dtype=np.float64)
    ys = xs if ys is None else np.asarray(ys, dtype=np.float64)
    n = xt.shape[0]
    keep = _mask(n, yt.shape[0], causal)

    # Item 1: logits of both models, masked.
    zt = np.where(keep, scale * (xt @ yt.T), _NEG_INF)
    zs = np.where(keep, scale * (xs @ ys.T), _NEG_INF)
    # Item 3: per-row log-partition.
    lse_t = _logsumexp_rows(zt)
    lse_s = _logsumexp_rows(zs)
    # Row-softmax maps in log form and probability form; masked entries are 0.
    # (Masked entries are set to log-probability 0 and probability 0, so they
    # add nothing below.)
    logr_t = np.where(keep, zt - lse_t[:, None], 0.0)
    logr_s = np.where(keep, zs - lse_s[:, None], 0.0)
    r_t = np.where(keep, np.exp(logr_t), 0.0)
    r_s = np.where(keep, np.exp(logr_s), 0.0)
    # Item 1: forward KL(R_t || R_s) per row; 0*log0 := 0 through the mask.
    row_kl = np.sum(r_t * (logr_t - logr_s), axis=1)
    loss = float(np.sum(row_kl) / n) if n else 0.0
    # Item 3: analytic logit gradient and its two contractions.
    dz = np.where(keep, r_s - r_t, 0.0) / max(n, 1)
    dxs = scale * (dz @ ys)
    dys = scale * (dz.T @ xs)
    return {"lse_t": lse_t, "lse_s": lse_s, "row_kl": row_kl, "loss": loss,
            "dz": dz, "dxs": dxs, "dys": dys, "dself": dxs + dys}


def relation_kl(xt: np.ndarray, xs: np.ndarray, scale: float, causal: bool = True,
                loss_scale: float = 1.0) -> Dict[str, np.ndarray]:
    """Self-relation KL over a [B, H, n, d] batch: per-head dense oracle, heads summed.

    Returns loss (float), lse_t/lse_s/row_kl [B, H, n] and dxs [B, H, n, d]
    (the total student gradient, already multiplied by loss_scale).
    """
    xt = np.asarray(xt, dtype=np.float64)
    xs = np.asarray(xs, dtype=np.float64)
    B, H, n, d = xt.shape
    lse_t = np.zeros((B, H, n)); lse_s = np.zeros((B, H, n)); row_kl = np.zeros((B, H, n))
    dxs = np.zeros((B, H, n, d))
    loss = 0.0
    for b in range(B):
        for h in range(H):
            r = relation_kl_head(xt[b, h], xs[b, h], scale, causal)
            lse_t[b, h], lse_s[b, h], row_kl[b, h] = r["lse_t"], r["lse_s"], r["row_kl"]
            dxs[b, h] = r["dself"] * loss_scale
            loss += r["loss"]
    return {"loss": loss * loss_scale, "lse_t": lse_t, "lse_s": lse_s,
            "row_kl": row_kl, "dxs": dxs}


def relation_kl_xy(xt: np.ndarray, xs: np.ndarray, yt: np.ndarray, ys: np.ndarray, scale: float,
                   causal: bool = True, loss_scale: float = 1.0) -> Dict[str, np.ndarray]:
    """General relation Z = scale * X Y^T over a [B, H, n, d] batch (notes page,
    "Key designs" item 1 for projected sequences X_m, Y_m; item 3 for the two
    contractions dX_s = scale*dZ Y_s and dY_s = scale*dZ^T X_s).

    Returns loss (heads summed, times loss_scale), lse_t/lse_s/row_kl [B,H,n],
    dxs and dys [B,H,n,d] (times loss_scale), from the dense per-head definition.
    """
    xt, xs, yt, ys = (np.asarray(v, dtype=np.float64) for v in (xt, xs, yt, ys))
    B, H, n, d = xt.shape
    out = {k: np.zeros((B, H, n)) for k in ("lse_t", "lse_s", "row_kl")}
    dxs = np.zeros((B, H, n, d))
    dys = np.zeros((B, H, n, d))
    loss = 0.0
    for b in range(B):
        for h in range(H):
            r = relation_kl_head(xt[b, h], xs[b, h], scale, causal, yt[b, h], ys[b, h])
            for k in ("lse_t", "lse_s", "row_kl"):
                out[k][b, h] = r[k]
            dxs[b, h] = r["dxs"] * loss_scale
            dys[b, h] = r["dys"] * loss_scale
            loss += r["loss"]
    return {"loss": loss * loss_scale, "dxs": dxs, "dys": dys, **out}


# ----------------------------------------------------------------------------
# Row-sampled forms of the same definitions, for sizes where a dense n x n map
# does not fit host memory.  Each output row is computed directly from its
# definition (one matrix product per block of requested rows); nothing is
# reordered inside a row.
# ----------------------------------------------------------------------------

def lse_rows(x: np.ndarray, scale: float, rows: Iterable[int], causal: bool = True,
             y: Optional[np.ndarray] = None) -> np.ndarray:
    """LSE(i) = log sum_{j kept} exp(scale <x_i, y_j>) for the requested rows."""
    x = np.asarray(x, dtype=np.float64)
    y = x if y is None else np.asarray(y, dtype=np.float64)
    rows = np.asarray(list(rows), dtype=np.int64)
    z = scale * (x[rows] @ y.T)
    if causal:
        z = np.where(np.arange(y.shape[0])[None, :] <= rows[:, None], z, _NEG_INF)
    return _logsumexp_rows(z)


def row_kl_rows(xt: np.ndarray, xs: np.ndarray, scale: float, rows: Iterable[int],
                causal: bool = True, yt: Optional[np.ndarray] = None,
                ys: Optional[np.ndarray] = None) -> np.ndarray:
    """KL(R_t(i,:) || R_s(i,:)) for the requested rows (Y = X unless given)."""
    xt = np.asarray(xt, dtype=np.float64)
    xs = np.asarray(xs, dtype=np.float64)
    yt = xt if yt is None else np.asarray(yt, dtype=np.float64)
    ys = xs if ys is None else np.asarray(ys, dtype=np.float64)
    rows = np.asarray(list(rows), dtype=np.int64)
    n = yt.shape[0]
    keep = (np.arange(n)[None, :] <= rows[:, None]) if causal else np.ones((len(rows), n), bool)
    zt = np.where(keep, scale * (xt[rows] @ yt.T), _NEG_INF)
    zs = np.where(keep, scale * (xs[rows] @ ys.T), _NEG_INF)
    logr_t = np.where(keep, zt - _logsumexp_rows(zt)[:, None], 0.0)
    logr_s = np.where(keep, zs - _logsumexp_rows(zs)[:, None], 0.0)
    r_t = np.where(keep, np.exp(logr_t), 0.0)
    return np.sum(r_t * (logr_t - logr_s), axis=1)


def dx_rows(xt: np.ndarray, xs: np.ndarray, scale: float, rows: Iterable[int],
            lse_t: np.ndarray, lse_s: np.ndarray, causal: bool = True) -> np.ndarray:
    """Total student gradient rows dX_s[i] = scale*(sum_j dZ(i,j) x_j + sum_j dZ(j,i) x_j).

    `lse_t`/`lse_s` are the oracle's own LSE over ALL rows (from `lse_rows`),
    needed because column i of dZ involves every row j >= i.
    """
    xt = np.asarray(xt, dtype=np.float64)
    xs = np.asarray(xs, dtype=np.float64)
    rows = np.asarray(list(rows), dtype=np.int64)
    n = xt.shape[0]
    cols = np.arange(n)
    # Row term: entries (i, j) of dZ.
    keep_r = (cols[None, :] <= rows[:, None]) if causal else np.ones((len(rows), n), bool)
    rt = np.where(keep_r, np.exp(np.where(keep_r, scale * (xt[rows] @ xt.T) - lse_t[rows][:, None], 0.0)), 0.0)
    rs = np.where(keep_r, np.exp(np.where(keep_r, scale * (xs[rows] @ xs.T) - lse_s[rows][:, None], 0.0)), 0.0)
    row_term = ((rs - rt) / n) @ xs
    # Column term: entries (j, i) of dZ, i.e. row j's probability of column i.
    keep_c = (cols[None, :] >= rows[:, None]) if causal else np.ones((len(rows), n), bool)
    ct = np.where(keep_c, np.exp(np.where(keep_c, scale * (xt[rows] @ xt.T) - lse_t[None, :], 0.0)), 0.0)
    cs = np.where(keep_c, np.exp(np.where(keep_c, scale * (xs[rows] @ xs.T) - lse_s[None, :], 0.0)), 0.0)
    col_term = ((cs - ct) / n) @ xs
    return scale * (row_term + col_term)


def dx_rows_xy(xt: np.ndarray, xs: np.ndarray, yt: np.ndarray, ys: np.ndarray, scale: float,
               rows: Iterable[int], lse_t: np.ndarray, lse_s: np.ndarray,
               causal: bool = True) -> np.ndarray:
    """Rows of dX_s = scale * dZ Y_s of an X/Y relation: sum_j dZ(i,j) y_s[j].

    `lse_t`/`lse_s`: the oracle's LSE of the requested rows (or of all rows).
    """
    xt, xs, yt, ys = (np.asarray(v, dtype=np.float64) for v in (xt, xs, yt, ys))
    rows = np.asarray(list(rows), dtype=np.int64)
    n = yt.shape[0]
    lt = np.asarray(lse_t)[rows] if len(lse_t) == n else np.asarray(lse_t)
    ls = np.asarray(lse_s)[rows] if len(lse_s) == n else np.asarray(lse_s)
    keep = (np.arange(n)[None, :] <= rows[:, None]) if causal else np.ones((len(rows), n), bool)
    rt = np.where(keep, np.exp(np.where(keep, scale * (xt[rows] @ yt.T) - lt[:, None], 0.0)), 0.0)
    rs = np.where(keep, np.exp(np.where(keep, scale * (xs[rows] @ ys.T) - ls[:, None], 0.0)), 0.0)
    return scale * (((rs - rt) / n) @ ys)


def dy_rows_xy(xt: np.ndarray, xs: np.ndarray, yt: np.ndarray, ys: np.ndarray, scale: float,
               cols: Iterable[int], lse_t: np.ndarray, lse_s: np.ndarray,
               causal: bool = True) -> np.ndarray:
    """Rows j of dY_s = scale * dZ^T X_s of an X/Y relation: sum_i dZ(i,j) x_s[i].

    Column j of dZ involves every row i (i >= j when causal), so `lse_t`/`lse_s`
    are the oracle's LSE over ALL rows (from `lse_rows`).
    """
    xt, xs, yt, ys = (np.asarray(v, dtype=np.float64) for v in (xt, xs, yt, ys))
    cols = np.asarray(list(cols), dtype=np.int64)
    n = xt.shape[0]
    keep = (np.arange(n)[None, :] >= cols[:, None]) if causal else np.ones((len(cols), n), bool)
    # entries (i, j) of Z for the requested j, laid out as [j, i]
    ct = np.where(keep, np.exp(np.where(keep, scale * (yt[cols] @ xt.T) - np.asarray(lse_t)[None, :], 0.0)), 0.0)
    cs = np.where(keep, np.exp(np.where(keep, scale * (ys[cols] @ xs.T) - np.asarray(lse_s)[None, :], 0.0)), 0.0)
    return scale * (((cs - ct) / n) @ xs)


# ----------------------------------------------------------------------------
# Projection backward (notes page, "Method details -> Overall framework" and
# "Loss function / training strategy": stage 1 updates only the attention
# projections).  X_s[b,h,i,:] = R(i) (h[b,i,:] W[:, h*d:(h+1)*d]) with R(i)
# the student's rotate-half rotation, so dW = h^T (R^T dX_s).
# ----------------------------------------------------------------------------

def rope_rotate(x: np.ndarray, cos: np.ndarray, sin: np.ndarray) -> np.ndarray:
    """Rotate-half rotation of [..., n, d]: pair (k, k+d/2) turned by the angle
    whose cos/sin are cos[i, k], sin[i, k] ([n, d/2] tables)."""
    x = np.asarray(x, dtype=np.float64)
    half = x.shape[-1] // 2
    x1, x2 = x[..., :half], x[..., half:]
    c, s = np.asarray(cos, np.float64), np.asarray(sin, np.float64)
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def rope_rotate_transpose(g: np.ndarray, cos: np.ndarray, sin: np.ndarray) -> np.ndarray:
    """R(i)^T applied to [..., n, d] (the rotation by the opposite angle)."""
    g = np.asarray(g, dtype=np.float64)
    half = g.shape[-1] // 2
    g1, g2 = g[..., :half], g[..., half:]
    c, s = np.asarray(cos, np.float64), np.asarray(sin, np.float64)
    return np.concatenate([g1 * c + g2 * s, g2 * c - g1 * s], axis=-1)


def proj_bwd(h: np.ndarray, dxs: np.ndarray, cos: Optional[np.ndarray] = None,
             sin: Optional[np.ndarray] = None) -> np.ndarray:
    """dW [dm, H*d] = sum over (b, i) of h[b,i,:]^T (R(i)^T dX_s[b,:,i,:]) (heads side by side).

    h: [B, n, dm]; dxs: [B, H, n, d]; cos/sin: [n, d/2] tables or None (no rotation).
    """
    h = np.asarray(h, dtype=np.float64)
    g = np.asarray(dxs, dtype=np.float64) if cos is None else rope_rotate_transpose(dxs, cos, sin)
    B, H, n, d = g.shape
    gm = np.transpose(g, (0, 2, 1, 3)).reshape(B * n, H * d)
    return h.reshape(B * n, h.shape[-1]).T @ gm
