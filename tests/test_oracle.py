"""Pins of the fp64 oracle against facts that do not come from the oracle itself.

Every check here is independent of the oracle's own code path: Gibbs'
inequality, special cases, finite differences, a probability-domain brute
force, a two-token closed form, a library (torch autograd) formulation, the
forward-KL small-probability limit of the notes page ("Key designs", item 2)
and orthogonal invariance.
"""
import math

import numpy as np
import pytest

import oracle
import synth_inputs as si

RNG = np.random.default_rng(1234)


def _pair(n, d, noise=0.3, seed=0):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((n, d))
    return x, x + noise * rng.standard_normal((n, d))


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("n,d", [(1, 4), (7, 3), (40, 16)])
def test_kl_nonnegative(n, d, causal):
    xt, xs = _pair(n, d, 1.0, seed=n)
    r = oracle.relation_kl_head(xt, xs, 0.4, causal)
    assert np.all(r["row_kl"] >= -1e-14)
    assert r["loss"] >= 0.0


@pytest.mark.parametrize("causal", [True, False])
def test_identical_inputs_give_exact_zero(causal):
    xt, _ = _pair(33, 8)
    r = oracle.relation_kl_head(xt, xt.copy(), 0.3, causal)
    assert r["loss"] == 0.0
    assert np.all(r["row_kl"] == 0.0)
    assert np.all(r["dself"] == 0.0)


def test_causal_row0_and_single_token():
    xt, xs = _pair(9, 5, 1.0)
    r = oracle.relation_kl_head(xt, xs, 0.5, True)
    assert r["row_kl"][0] == 0.0
    assert np.all(r["dz"][0] == 0.0)
    # row 0's only probability is 1 for both models
    assert r["lse_t"][0] == pytest.approx(0.5 * xt[0] @ xt[0], abs=1e-14)
    r1 = oracle.relation_kl_head(xt[:1], xs[:1], 0.5, True)
    assert r1["loss"] == 0.0 and np.all(r1["dself"] == 0.0)


@pytest.mark.parametrize("causal", [True, False])
def test_dz_rows_sum_to_zero(causal):
    xt, xs = _pair(50, 6, 1.0)
    r = oracle.relation_kl_head(xt, xs, 0.45, causal)
    assert np.max(np.abs(r["dz"].sum(axis=1))) < 1e-16


def _fd_grad(f, x, h=1e-6):
    g = np.zeros_like(x)
    for idx in np.ndindex(x.shape):
        xp = x.copy(); xp[idx] += h
        xm = x.copy(); xm[idx] -= h
        g[idx] = (f(xp) - f(xm)) / (2 * h)
    return g


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("n,d,s", [(12, 4, 0.5), (33, 3, 0.9)])
def test_gradient_matches_central_differences(n, d, s, causal):
    xt, xs = _pair(n, d, 0.7, seed=n + d)
    r = oracle.relation_kl_head(xt, xs, s, causal)
    fd = _fd_grad(lambda v: oracle.relation_kl_head(xt, v, s, causal)["loss"], xs)
    err = np.max(np.abs(fd - r["dself"])) / np.max(np.abs(fd))
    assert err < 1e-7, err


def test_cross_relation_gradients_match_central_differences():
    # General X != Y form (dX_s and dY_s of "Key designs" item 3).
    rng = np.random.default_rng(5)
    n, d, s = 10, 4, 0.6
    xt, yt = rng.standard_normal((n, d)), rng.standard_normal((n, d))
    xs, ys = xt + 0.5 * rng.standard_normal((n, d)), yt + 0.5 * rng.standard_normal((n, d))
    r = oracle.relation_kl_head(xt, xs, s, True, yt=yt, ys=ys)
    fx = _fd_grad(lambda v: oracle.relation_kl_head(xt, v, s, True, yt=yt, ys=ys)["loss"], xs)
    fy = _fd_grad(lambda v: oracle.relation_kl_head(xt, xs, s, True, yt=yt, ys=v)["loss"], ys)
    assert np.max(np.abs(fx - r["dxs"])) / np.max(np.abs(fx)) < 1e-7
    assert np.max(np.abs(fy - r["dys"])) / np.max(np.abs(fy)) < 1e-7


def _brute_kl(xt, xs, s, causal):
    """Probability-domain KL with explicit loops: p = e^z / sum e^z, KL = sum p log(p/q)."""
    n = len(xt)
    out = []
    for i in range(n):
        cols = range(i + 1) if causal else range(n)
        et = [math.exp(s * float(np.dot(xt[i], xt[j]))) for j in cols]
        es = [math.exp(s * float(np.dot(xs[i], xs[j]))) for j in cols]
        zt, zs = sum(et), sum(es)
        kl = 0.0
        for a, b in zip(et, es):
            p, q = a / zt, b / zs
            if p > 0:
                kl += p * math.log(p / q)
        out.append(kl)
    return np.array(out)


@pytest.mark.parametrize("causal", [True, False])
def test_bruteforce_probability_domain(causal):
    xt, xs = _pair(8, 3, 0.8, seed=3)
    r = oracle.relation_kl_head(xt, xs, 0.7, causal)
    bk = _brute_kl(xt, xs, 0.7, causal)
    assert np.max(np.abs(bk - r["row_kl"])) < 1e-13
    assert r["loss"] == pytest.approx(bk.sum() / 8, rel=1e-12)


@pytest.mark.parametrize("vals", [(0.3, 1.1, -0.4, 0.9, 0.8), (1.5, -0.7, 1.2, 0.2, 0.35)])
def test_two_token_closed_form(vals):
    # n=2, d=1, causal: row 1 has logits [s x1 x0, s x1^2]; row 0 is trivial.
    x0t, x1t, x0s, x1s, s = vals
    sig = lambda u: 1.0 / (1.0 + math.exp(-u))
    p = sig(s * x1t * (x1t - x0t))
    q = sig(s * x1s * (x1s - x0s))
    kl1 = p * math.log(p / q) + (1 - p) * math.log((1 - p) / (1 - q))
    r = oracle.relation_kl_head(np.array([[x0t], [x1t]]), np.array([[x0s], [x1s]]), s, True)
    assert r["loss"] == pytest.approx(kl1 / 2, rel=1e-13, abs=1e-16)
    assert r["dself"][0, 0] == pytest.approx(s * (p - q) / 2 * x1s, rel=1e-12, abs=1e-16)
    assert r["dself"][1, 0] == pytest.approx(s * (q - p) / 2 * (2 * x1s - x0s), rel=1e-12, abs=1e-16)


def test_forward_kl_gradient_survives_vanishing_student_probability():
    # Notes page, "Key designs" item 2: as r_s -> 0 with r_t > 0 the logit
    # gradient tends to -r_t (here divided by the row count n = 2).
    s = 1.0
    xt = np.array([[1.0], [1.0]])          # teacher row 1: p = 1/2 on both columns
    x0s = -5.0                               # student: r_s(1, 0) = sigmoid(-x1 (x1 - x0))
    x1s = (x0s + math.sqrt(x0s ** 2 + 4 * 27.6)) / 2      # x1 (x1 - x0) = 27.6
    r = oracle.relation_kl_head(xt, np.array([[x0s], [x1s]]), s, True)
    rs10 = 1.0 / (1.0 + math.exp(27.6))
    assert rs10 < 1e-11
    assert r["dz"][1, 0] == pytest.approx((rs10 - 0.5) / 2, abs=1e-15)
    assert r["dz"][1, 0] == pytest.approx(-0.5 / 2, abs=1e-11)


def test_orthogonal_invariance():
    xt, xs = _pair(25, 6, 0.6, seed=9)
    q, _ = np.linalg.qr(np.random.default_rng(2).standard_normal((6, 6)))
    a = oracle.relation_kl_head(xt, xs, 0.5, True)
    b = oracle.relation_kl_head(xt @ q, xs @ q, 0.5, True)
    assert b["loss"] == pytest.approx(a["loss"], rel=1e-12)
    assert np.max(np.abs(b["dself"] - a["dself"] @ q)) < 1e-14


def test_vanishing_scale_gives_uniform_rows_and_zero_loss():
    xt, xs = _pair(20, 4, 2.0)
    r = oracle.relation_kl_head(xt, xs, 1e-9, True)
    assert r["loss"] < 1e-15
    n = 20
    assert np.allclose(r["lse_t"], np.log(np.arange(1, n + 1)), atol=1e-7)


@pytest.mark.parametrize("causal", [True, False])
def test_agrees_with_torch_autograd(causal):
    torch = pytest.importorskip("torch")
    xt, xs = _pair(30, 5, 0.5, seed=11)
    s = 0.45
    Xt = torch.tensor(xt, dtype=torch.float64)
    Xs = torch.tensor(xs, dtype=torch.float64, requires_grad=True)
    zt, zs = s * Xt @ Xt.T, s * Xs @ Xs.T
    if causal:
        m = torch.ones(30, 30, dtype=torch.bool).tril()
        zt = zt.masked_fill(~m, -1e30)
        zs = zs.masked_fill(~m, -1e30)
    lt = torch.log_softmax(zt, dim=1)
    ls = torch.log_softmax(zs, dim=1)
    loss = torch.nn.functional.kl_div(ls, lt, reduction="sum", log_target=True) / 30
    loss.backward()
    r = oracle.relation_kl_head(xt, xs, s, causal)
    assert float(loss.detach()) == pytest.approx(r["loss"], rel=1e-12)
    assert np.max(np.abs(Xs.grad.numpy() - r["dself"])) < 1e-15 + 1e-12 * np.max(np.abs(r["dself"]))


def test_batched_sum_and_loss_scale():
    rng = np.random.default_rng(3)
    xt = rng.standard_normal((2, 3, 11, 4)); xs = xt + 0.4 * rng.standard_normal(xt.shape)
    out = oracle.relation_kl(xt, xs, 0.5, True, loss_scale=0.25)
    tot = 0.0
    for b in range(2):
        for h in range(3):
            r = oracle.relation_kl_head(xt[b, h], xs[b, h], 0.5, True)
            tot += r["loss"]
            assert np.array_equal(out["dxs"][b, h], 0.25 * r["dself"])
    assert out["loss"] == pytest.approx(0.25 * tot, rel=1e-15)


@pytest.mark.parametrize("causal", [True, False])
def test_row_sampled_forms_match_dense(causal):
    xt, xs = _pair(45, 7, 0.5, seed=21)
    s = 0.4
    r = oracle.relation_kl_head(xt, xs, s, causal)
    rows = [0, 1, 17, 44]
    lt = oracle.lse_rows(xt, s, range(45), causal)
    ls = oracle.lse_rows(xs, s, range(45), causal)
    assert np.max(np.abs(lt - r["lse_t"])) < 1e-13
    assert np.max(np.abs(oracle.row_kl_rows(xt, xs, s, rows, causal) - r["row_kl"][rows])) < 1e-14
    got = oracle.dx_rows(xt, xs, s, rows, lt, ls, causal)
    assert np.max(np.abs(got - r["dself"][rows])) < 1e-15


# ---------------------------------------------------------------------------
# General relation X != Y (notes page, "Key designs" items 1 and 3).
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("vals", [(0.3, 1.1, -0.4, 0.9, 0.7, -0.2, 1.3, 0.6, 0.8),
                                  (1.5, -0.7, 1.2, 0.2, -0.9, 0.4, 0.1, 1.1, 0.35)])
def test_cross_two_token_closed_form(vals):
    # n=2, d=1, causal.  Row 1 has logits [s x1 y0, s x1 y1], so
    # r(1,1) = sigmoid(s x1 (y1 - y0)); row 0 is the single entry (0,0).
    x0t, x1t, x0s, x1s, y0t, y1t, y0s, y1s, s = vals
    sig = lambda u: 1.0 / (1.0 + math.exp(-u))
    p = sig(s * x1t * (y1t - y0t))
    q = sig(s * x1s * (y1s - y0s))
    kl1 = p * math.log(p / q) + (1 - p) * math.log((1 - p) / (1 - q))
    r = oracle.relation_kl_head(np.array([[x0t], [x1t]]), np.array([[x0s], [x1s]]), s, True,
                                np.array([[y0t], [y1t]]), np.array([[y0s], [y1s]]))
    assert r["loss"] == pytest.approx(kl1 / 2, rel=1e-13, abs=1e-16)
    # dZ(1,1) = (q - p)/2, dZ(1,0) = (p - q)/2, dZ(0,0) = 0
    assert r["dxs"][0, 0] == pytest.approx(0.0, abs=1e-16)
    assert r["dxs"][1, 0] == pytest.approx(s * (q - p) / 2 * (y1s - y0s), rel=1e-12, abs=1e-16)
    assert r["dys"][0, 0] == pytest.approx(s * (p - q) / 2 * x1s, rel=1e-12, abs=1e-16)
    assert r["dys"][1, 0] == pytest.approx(s * (q - p) / 2 * x1s, rel=1e-12, abs=1e-16)


def test_cross_with_y_equal_x_is_the_self_relation():
    rng = np.random.default_rng(31)
    xt = rng.standard_normal((2, 2, 13, 5)); xs = xt + 0.3 * rng.standard_normal(xt.shape)
    a = oracle.relation_kl_xy(xt, xs, xt, xs, 0.6, True, loss_scale=0.5)
    b = oracle.relation_kl(xt, xs, 0.6, True, loss_scale=0.5)
    assert a["loss"] == pytest.approx(b["loss"], rel=1e-14)
    assert np.max(np.abs(a["dxs"] + a["dys"] - b["dxs"])) < 1e-15
    assert np.array_equal(a["row_kl"], b["row_kl"])


def test_cross_kl_nonnegative_and_zero_for_identical_models():
    rng = np.random.default_rng(32)
    x = rng.standard_normal((1, 2, 20, 6)); y = rng.standard_normal((1, 2, 20, 6))
    r = oracle.relation_kl_xy(x, x + 0.5 * rng.standard_normal(x.shape), y, y, 0.5, True)
    assert np.all(r["row_kl"] > -1e-15)
    z = oracle.relation_kl_xy(x, x, y, y, 0.5, False)
    assert z["loss"] == 0.0 and np.all(z["dxs"] == 0.0) and np.all(z["dys"] == 0.0)


@pytest.mark.parametrize("causal", [True, False])
def test_cross_row_sampled_forms_match_dense(causal):
    rng = np.random.default_rng(33)
    n, d, s = 40, 6, 0.45
    xt = rng.standard_normal((n, d)); xs = xt + 0.4 * rng.standard_normal((n, d))
    yt = rng.standard_normal((n, d)); ys = yt + 0.4 * rng.standard_normal((n, d))
    r = oracle.relation_kl_head(xt, xs, s, causal, yt, ys)
    rows = [0, 1, 19, 39]
    lt = oracle.lse_rows(xt, s, range(n), causal, y=yt)
    ls = oracle.lse_rows(xs, s, range(n), causal, y=ys)
    assert np.max(np.abs(lt - r["lse_t"])) < 1e-13
    assert np.max(np.abs(oracle.row_kl_rows(xt, xs, s, rows, causal, yt, ys) - r["row_kl"][rows])) < 1e-14
    assert np.max(np.abs(oracle.dx_rows_xy(xt, xs, yt, ys, s, rows, lt, ls, causal) - r["dxs"][rows])) < 1e-15
    assert np.max(np.abs(oracle.dy_rows_xy(xt, xs, yt, ys, s, rows, lt, ls, causal) - r["dys"][rows])) < 1e-15


# ---------------------------------------------------------------------------
# Projection backward (dW = h^T R^T dX_s).
# ---------------------------------------------------------------------------
def _tables(n, d, base=1.0e4, pos_scale=2.0):
    c, s = si.rope_tables(n, d, base, pos_scale)
    return c[:, : d // 2], s[:, : d // 2]


def test_rope_rotation_transpose_and_generator_agree():
    rng = np.random.default_rng(41)
    n, d = 9, 8
    c, s = _tables(n, d)
    x = rng.standard_normal((2, 3, n, d))
    y = oracle.rope_rotate(x, c, s)
    assert np.max(np.abs(oracle.rope_rotate_transpose(y, c, s) - x)) < 1e-14      # R^T R = I
    assert np.allclose(np.sum(y ** 2, -1), np.sum(x ** 2, -1), rtol=1e-14)         # a rotation
    full_c, full_s = si.rope_tables(n, d, 1.0e4, 2.0)
    assert np.max(np.abs(y - si.apply_rope(x, full_c, full_s))) < 1e-14             # input convention
    # a unit pair at angle theta goes to (cos theta, sin theta)
    e = np.zeros((1, 1, n, d)); e[..., 0] = 1.0
    r = oracle.rope_rotate(e, c, s)
    assert np.allclose(r[0, 0, :, 0], c[:, 0]) and np.allclose(r[0, 0, :, d // 2], s[:, 0])


def test_proj_bwd_matches_finite_differences_through_rope_and_relation():
    # L(W) = relation KL of teacher X_t and student X_s = R (h W), per head.
    rng = np.random.default_rng(42)
    B, n, dm, H, d, scale = 1, 7, 5, 2, 4, 0.6
    c, s = _tables(n, d)
    h = rng.standard_normal((B, n, dm))
    W = rng.standard_normal((dm, H * d)) * 0.5
    xt = rng.standard_normal((B, H, n, d))

    def xs_of(Wm):
        p = (h @ Wm).reshape(B, n, H, d).transpose(0, 2, 1, 3)
        return oracle.rope_rotate(p, c, s)

    def loss(Wm):
        return oracle.relation_kl(xt, xs_of(Wm), scale, True)["loss"]

    dxs = oracle.relation_kl(xt, xs_of(W), scale, True)["dxs"]
    dW = oracle.proj_bwd(h, dxs, c, s)
    eps = 1e-6
    for (a, b) in [(0, 0), (1, 3), (4, 5), (2, 7), (3, 1)]:
        Wp, Wn = W.copy(), W.copy()
        Wp[a, b] += eps
        Wn[a, b] -= eps
        fd = (loss(Wp) - loss(Wn)) / (2 * eps)
        assert abs(fd - dW[a, b]) < 1e-7 * max(1.0, abs(dW[a, b])), (a, b, fd, dW[a, b])


def test_proj_bwd_without_rotation_is_a_plain_product():
    rng = np.random.default_rng(43)
    h = rng.standard_normal((2, 5, 3)); g = rng.standard_normal((2, 2, 5, 4))
    got = oracle.proj_bwd(h, g)
    want = np.zeros((3, 8))
    for b in range(2):
        for i in range(5):
            for hd in range(2):
                want[:, hd * 4:(hd + 1) * 4] += np.outer(h[b, i], g[b, hd, i])
    assert np.max(np.abs(got - want)) < 1e-14
