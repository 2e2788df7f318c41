"""GPU parity of the general relation X != Y (Z = s X Y^T) against the fp64 oracle.

Same bars as the self-relation: bf16 inputs 1e-3 on the loss and 2e-2
normwise max-relative on each of dX_s and dY_s; fp32 inputs 1e-5.  LSE and
row KL are compared with the bounds derived from fp32 accumulation.
"""
import numpy as np
import pytest

import oracle
import synth_inputs as si
from helpers import normwise_max_rel, rel, to_device, widen

pytestmark = pytest.mark.gpu

TOL = {"f32": dict(loss=1e-5, dx=1e-5, lse=1e-9, kl=1e-7),
       "bf16": dict(loss=1e-3, dx=2e-2, lse=2e-6, kl=2e-6)}
EPS32 = 2.0 ** -24


def f32(v):
    return float(np.float32(v))


def _quad(B, H, n, d, noise, seed, dtype="bf16"):
    """Teacher/student X and Y: Y independent of X, students perturbed."""
    rng = np.random.default_rng(seed)
    xt = rng.standard_normal((B, H, n, d))
    yt = rng.standard_normal((B, H, n, d))
    xs = xt + noise * rng.standard_normal(xt.shape)
    ys = yt + noise * rng.standard_normal(yt.shape)
    rnd = si.round_bf16_bits if dtype == "bf16" else si.round_f32
    return tuple(rnd(v) for v in (xt, xs, yt, ys))


def _zmax(a, b, c, e, s):
    """Bound on |logit|: s * max|x| * max|y| (Cauchy-Schwarz), for either model."""
    nx = max(np.max(np.linalg.norm(a, axis=-1)), np.max(np.linalg.norm(b, axis=-1)))
    ny = max(np.max(np.linalg.norm(c, axis=-1)), np.max(np.linalg.norm(e, axis=-1)))
    return s * nx * ny


def _run(lmr, arrs, dtype, scale, causal=True, loss_scale=1.0):
    import torch
    xt, xs, yt, ys = (to_device(v, dtype) for v in arrs)
    lt, ls = lmr.xy_lse_fwd(xt, xs, yt, ys, scale, causal)
    rk, dx, dy = lmr.xy_kl_bwd(xt, xs, yt, ys, lt, ls, scale, causal, loss_scale)
    loss, dx2, dy2 = lmr.xy_loss(xt, xs, yt, ys, scale, causal, loss_scale)
    f_lt, f_ls, f_kl = lmr.xy_kl_fwd(xt, xs, yt, ys, scale, causal)
    _, dx3, _ = lmr.xy_kl_bwd(xt, xs, yt, ys, lt, ls, scale, causal, loss_scale, need_dy=False)
    _, _, dy3 = lmr.xy_kl_bwd(xt, xs, yt, ys, lt, ls, scale, causal, loss_scale, need_dx=False)
    torch.cuda.synchronize()
    c = lambda t: t.cpu().numpy()
    return dict(lse_t=c(lt), lse_s=c(ls), row_kl=c(rk), dx=c(dx), dy=c(dy), loss=float(loss.cpu()),
                dx2=c(dx2), dy2=c(dy2), dx3=c(dx3), dy3=c(dy3), f_lt=c(f_lt), f_ls=c(f_ls), f_kl=c(f_kl))


def _compare(got, ref, dtype, zmax, n, loss_scale=1.0, s=None, ymax=None):
    tol = TOL[dtype]
    scale_err = (EPS32 * zmax * 8) if dtype == "bf16" else 0.0
    for k, fk in (("lse_t", "f_lt"), ("lse_s", "f_ls")):
        bound = tol["lse"] * (1 + np.max(np.abs(ref[k]))) + scale_err
        assert np.max(np.abs(got[k] - ref[k])) < bound, k
        assert np.max(np.abs(got[fk] - ref[k])) < bound, fk
    kl_bound = tol["kl"] + 1e-4 * np.max(np.abs(ref["row_kl"])) + scale_err
    assert np.max(np.abs(got["row_kl"] - ref["row_kl"])) < kl_bound
    assert np.max(np.abs(got["f_kl"] - ref["row_kl"])) < kl_bound
    if abs(ref["loss"]) > 1e-4 * loss_scale:
        assert rel(got["loss"], ref["loss"]) < tol["loss"], (got["loss"], ref["loss"])
    else:
        assert abs(got["loss"] - ref["loss"]) < kl_bound * loss_scale
    for k, rk in (("dx", "dxs"), ("dy", "dys")):
        e = normwise_max_rel(got[k], ref[rk])
        if n <= 8 and dtype == "bf16":
            # Degenerate lengths: the gradient can be ~1e-6 of its terms; bound
            # by the relative error eps_p of each recomputed probability.
            eps_p = 4 * EPS32 * (1 + 1.4427 * max(np.max(np.abs(ref["lse_t"])), np.max(np.abs(ref["lse_s"]))))
            bound = loss_scale * s / n * eps_p * (2 + n) * ymax
            assert e < tol["dx"] or np.max(np.abs(got[k] - ref[rk])) < bound, (k, e, bound)
        else:
            assert e < tol["dx"], (k, e)
    # one-call path and single-gradient calls reproduce the two-call path bit for bit
    for a, b in (("dx", "dx2"), ("dy", "dy2"), ("dx", "dx3"), ("dy", "dy3")):
        assert np.array_equal(got[a], got[b]), (a, b)


@pytest.mark.parametrize("n", [1, 2, 31, 64, 65, 129, 200, 257, 333, 513])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [True, False])
def test_xy_bf16_ragged(gpu_lib, n, d, causal):
    arrs = _quad(1, 2, n, d, 0.4, seed=7 * n + d + causal)
    s = 1.0 / np.sqrt(d)
    got = _run(gpu_lib, arrs, "bf16", s, causal)
    w = [widen(v, "bf16") for v in arrs]
    ref = oracle.relation_kl_xy(*w, f32(s), causal)
    ymax = max(float(np.max(np.abs(w[1]))), float(np.max(np.abs(w[3]))))
    _compare(got, ref, "bf16", _zmax(*w, s), n, s=s, ymax=ymax)


@pytest.mark.parametrize("n,causal", [(1, True), (100, True), (130, False)])
def test_xy_fp32(gpu_lib, n, causal):
    arrs = _quad(2, 1, n, 64, 0.4, seed=50 + n, dtype="f32")
    s = 0.125
    got = _run(gpu_lib, arrs, "f32", s, causal)
    w = [widen(v, "f32") for v in arrs]
    ref = oracle.relation_kl_xy(*w, f32(s), causal)
    _compare(got, ref, "f32", _zmax(*w, s), n)


def test_xy_multi_batch_loss_scale(gpu_lib):
    arrs = _quad(2, 3, 190, 128, 0.3, seed=61)
    s = 1.0 / np.sqrt(128)
    got = _run(gpu_lib, arrs, "bf16", s, True, loss_scale=1.0 / 6)
    w = [widen(v, "bf16") for v in arrs]
    ref = oracle.relation_kl_xy(*w, f32(s), True, loss_scale=1.0 / 6)
    _compare(got, ref, "bf16", _zmax(*w, s), 190, loss_scale=1.0 / 6)


def test_xy_identical_models_give_exact_zero(gpu_lib):
    xt, _, yt, _ = _quad(1, 2, 260, 128, 0.0, seed=62)
    got = _run(gpu_lib, (xt, xt.copy(), yt, yt.copy()), "bf16", 1 / np.sqrt(128))
    assert got["loss"] == 0.0 and np.all(got["row_kl"] == 0.0) and np.all(got["f_kl"] == 0.0)
    assert np.all(got["dx"] == 0.0) and np.all(got["dy"] == 0.0)


def test_xy_with_y_equal_x_matches_the_self_relation(gpu_lib):
    import torch
    xt, xs, _, _ = _quad(1, 2, 300, 128, 0.3, seed=63)
    a, b = to_device(xt, "bf16"), to_device(xs, "bf16")
    s = 1.0 / np.sqrt(128)
    loss_xy, dx, dy = gpu_lib.xy_loss(a, b, a, b, s, True)
    loss_self, dself = gpu_lib.loss(a, b, s, True)
    torch.cuda.synchronize()
    assert rel(float(loss_xy.cpu()), float(loss_self.cpu())) < 1e-6
    ref = oracle.relation_kl(widen(xt, "bf16"), widen(xs, "bf16"), f32(s), True)["dxs"]
    assert normwise_max_rel((dx + dy).cpu().numpy(), ref) < 2e-2
    assert normwise_max_rel(dself.cpu().numpy(), ref) < 2e-2


@pytest.mark.parametrize("causal", [True, False])
def test_xy_overflowing_shift_takes_the_exact_fallback(gpu_lib, causal):
    # Key 5 has a huge norm: for later queries its logit exceeds the diagonal
    # logit by far more than fp32 exp2 can hold.
    n, d = 150, 64
    rng = np.random.default_rng(64)
    xt = rng.standard_normal((1, 2, n, d)); yt = rng.standard_normal((1, 2, n, d))
    yt[:, :, 5] *= 40.0
    xs = xt + 0.3 * rng.standard_normal(xt.shape); ys = yt + 0.3 * rng.standard_normal(yt.shape)
    arrs = tuple(si.round_bf16_bits(v) for v in (xt, xs, yt, ys))
    got = _run(gpu_lib, arrs, "bf16", 0.125, causal)
    w = [widen(v, "bf16") for v in arrs]
    ref = oracle.relation_kl_xy(*w, 0.125, causal)
    assert all(np.all(np.isfinite(got[k])) for k in ("lse_t", "dx", "dy", "f_kl"))
    _compare(got, ref, "bf16", _zmax(*w, 0.125), n)


def test_xy_query_key_relation_of_rope_inputs(gpu_lib):
    # The query/key attention map of the LLaMA2-shaped inputs (X = Q, Y = K).
    w = si.workload("llama2_4k", n=320)
    maps = si.make_inputs(w, maps=["Q", "K"])
    q, k = maps["Q"], maps["K"]
    sl = lambda a: np.ascontiguousarray(a[:, :3])
    arrs = (sl(q.xt), sl(q.xs), sl(k.xt), sl(k.xs))
    got = _run(gpu_lib, arrs, "bf16", w.scale, True)
    wide = [q.xt64[:, :3], q.xs64[:, :3], k.xt64[:, :3], k.xs64[:, :3]]
    ref = oracle.relation_kl_xy(*wide, f32(w.scale), True)
    _compare(got, ref, "bf16", _zmax(*wide, w.scale), 320)
