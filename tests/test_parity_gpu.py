"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Tolerances: fp32 inputs 1e-5 (loss relative, gradient normwise max-relative);
bf16 inputs 1e-3 on the loss and 2e-2 on the gradient.  LSE and per-row KL
are compared elementwise with bounds derived from fp32 accumulation.
"""
import numpy as np
import pytest

import oracle
import synth_inputs as si
from helpers import normwise_max_rel, random_pair, rel, to_device, widen

pytestmark = pytest.mark.gpu

TOL = {"f32": dict(loss=1e-5, dx=1e-5, lse=1e-9, kl=1e-7),
       "bf16": dict(loss=1e-3, dx=2e-2, lse=2e-6, kl=2e-6)}
EPS32 = 2.0 ** -24


def _logit_bound(xt, xs, scale):
    """Largest |logit| the inputs can produce: scale * max_i |x_i|^2 (Cauchy-Schwarz)."""
    return scale * max(float(np.max(np.sum(xt ** 2, axis=-1))), float(np.max(np.sum(xs ** 2, axis=-1))))


def f32(v: float) -> float:
    """The scale as the C ABI receives it (a float argument); the oracle gets the same value."""
    return float(np.float32(v))


def _run(lmr, xt_np, xs_np, dtype, scale, causal=True, loss_scale=1.0, dx_mode=0):
    import torch
    xt, xs = to_device(xt_np, dtype), to_device(xs_np, dtype)
    lse_t, lse_s = lmr.lse_fwd(xt, xs, scale, causal)
    row_kl, dx = lmr.kl_bwd(xt, xs, lse_t, lse_s, scale, causal, loss_scale, dx_mode=dx_mode)
    loss, dx2 = lmr.loss(xt, xs, scale, causal, loss_scale, dx_mode=dx_mode)
    torch.cuda.synchronize()
    out = dict(lse_t=lse_t.cpu().numpy(), lse_s=lse_s.cpu().numpy(), row_kl=row_kl.cpu().numpy(),
               dx=dx.cpu().numpy(), loss=float(loss.cpu()), dx2=dx2.cpu().numpy())
    return out


def _compare(got, ref, dtype, n, zmax, loss_scale=1.0, scale=None, xmax=None):
    """zmax: bound on |logit| (nats); fp32 logits carry an absolute error ~eps32*zmax,
    which bounds what the LSE and per-row KL can resolve for bf16 inputs."""
    tol = TOL[dtype]
    scale_err = (EPS32 * zmax * 8) if dtype == "bf16" else 0.0
    for k in ("lse_t", "lse_s"):
        err = np.max(np.abs(got[k] - ref[k]))
        assert err < tol["lse"] * (1 + np.max(np.abs(ref[k]))) + scale_err, (k, err)
    kl_err = np.max(np.abs(got["row_kl"] - ref["row_kl"]))
    assert kl_err < tol["kl"] + 1e-4 * np.max(np.abs(ref["row_kl"])) + scale_err, kl_err
    if abs(ref["loss"]) > 1e-4 * loss_scale:
        assert rel(got["loss"], ref["loss"]) < tol["loss"], (got["loss"], ref["loss"])
    else:   # degenerate (near-)zero loss: absolute bound from the per-row KL bound
        assert abs(got["loss"] - ref["loss"]) < (tol["kl"] + scale_err) * loss_scale, (got["loss"], ref["loss"])
    e = normwise_max_rel(got["dx"], ref["dxs"])
    if n <= 8 and dtype == "bf16":
        # Degenerate lengths: the true gradient can be ~1e-6 of its terms, below
        # what fp32 statistics resolve.  Each recomputed probability carries a
        # relative error eps_p from the fp32 LSE and exp2; with at most n rows
        # per column, |d dX| <= loss_scale*scale/n * eps_p * (2 + n) * max|x_s|.
        eps_p = 4 * EPS32 * (1 + 1.4427 * max(np.max(np.abs(ref["lse_t"])), np.max(np.abs(ref["lse_s"]))))
        bound = loss_scale * scale / n * eps_p * (2 + n) * xmax
        assert e < tol["dx"] or np.max(np.abs(got["dx"] - ref["dxs"])) < bound, (e, bound)
    else:
        assert e < tol["dx"], e
    # the one-call path reproduces the two-call path bit for bit
    assert np.array_equal(got["dx"], got["dx2"])


def test_tiny_fp32_rope_pi4(gpu_lib):
    """Tiny fp32 Q/Q relation: n=256, d=64, PI x4 student (parity at 1e-5)."""
    w = si.WORKLOADS["tiny_f32"]
    m = si.make_inputs(w)["Q"]
    got = _run(gpu_lib, m.xt, m.xs, "f32", w.scale)
    ref = oracle.relation_kl(m.xt64, m.xs64, f32(w.scale), True)
    _compare(got, ref, "f32", w.n, _logit_bound(m.xt64, m.xs64, w.scale))


# Phase-2 modes of the bf16 path: FUSED (one sweep per row block) and SPLIT
# (row sweep, then column sweep; AUTO's choice).
MODES = [pytest.param(3, id="fused"), pytest.param(1, id="split")]


# Lengths around the 32-row block, the 128-row tile and the 256-row workgroup.
@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("n", [1, 2, 31, 63, 64, 65, 127, 128, 129, 200, 255, 256, 257, 333, 511, 513])
@pytest.mark.parametrize("d", [64, 128])
def test_bf16_ragged_lengths(gpu_lib, n, d, mode):
    xt, xs = random_pair(1, 2, n, d, 0.4, seed=n * 7 + d)
    s = 1.0 / np.sqrt(d)
    got = _run(gpu_lib, xt, xs, "bf16", s, dx_mode=mode)
    a, b = widen(xt, "bf16"), widen(xs, "bf16")
    ref = oracle.relation_kl(a, b, f32(s), True)
    _compare(got, ref, "bf16", n, _logit_bound(a, b, s), scale=s, xmax=float(np.max(np.abs(b))))


@pytest.mark.parametrize("n", [1, 65, 200])
@pytest.mark.parametrize("d", [64, 128])
def test_fp32_ragged_lengths(gpu_lib, n, d):
    xt, xs = random_pair(2, 1, n, d, 0.4, seed=n + d, dtype="f32")
    s = 1.0 / np.sqrt(d)
    got = _run(gpu_lib, xt, xs, "f32", s)
    a, b = widen(xt, "f32"), widen(xs, "f32")
    ref = oracle.relation_kl(a, b, f32(s), True)
    _compare(got, ref, "f32", n, _logit_bound(a, b, s))


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("n,d,dtype", [(200, 128, "bf16"), (129, 64, "bf16"), (100, 64, "f32"), (257, 64, "bf16"),
                                         (513, 128, "bf16")])
def test_bidirectional_mask(gpu_lib, n, d, dtype, mode):
    xt, xs = random_pair(1, 3, n, d, 0.5, seed=5, dtype=dtype)
    s = 1.0 / np.sqrt(d)
    got = _run(gpu_lib, xt, xs, dtype, s, causal=False, dx_mode=mode)
    a, b = widen(xt, dtype), widen(xs, dtype)
    ref = oracle.relation_kl(a, b, f32(s), False)
    _compare(got, ref, dtype, n, _logit_bound(a, b, s))


def test_multi_batch_heads_and_loss_scale(gpu_lib):
    B, H, n, d = 2, 3, 257, 128
    xt, xs = random_pair(B, H, n, d, 0.3, seed=11)
    s = 1.0 / np.sqrt(d)
    ls = 1.0 / (B * H)
    got = _run(gpu_lib, xt, xs, "bf16", s, loss_scale=ls)
    a, b = widen(xt, "bf16"), widen(xs, "bf16")
    ref = oracle.relation_kl(a, b, f32(s), True, loss_scale=ls)
    _compare(got, ref, "bf16", n, _logit_bound(a, b, s), loss_scale=ls)


def test_identical_inputs_give_exact_zero(gpu_lib):
    xt, _ = random_pair(1, 2, 300, 128, 0.0, seed=3)
    got = _run(gpu_lib, xt, xt.copy(), "bf16", 1 / np.sqrt(128))
    assert got["loss"] == 0.0
    assert np.all(got["row_kl"] == 0.0)
    assert np.all(got["dx"] == 0.0)


def test_single_token_and_empty(gpu_lib):
    import torch
    xt, xs = random_pair(1, 1, 1, 64, 1.0, seed=1)
    got = _run(gpu_lib, xt, xs, "bf16", 0.125)
    # One token: both rows are the single probability 1, so the exact loss and
    # gradient are 0; what is left is fp32 rounding of exp2/log2 near 1 (KL)
    # and of the two recomputed probabilities (gradient, relative eps_p).
    eps_p = 4 * EPS32 * (1 + 1.4427 * float(np.max(np.abs(got["lse_t"]))))
    assert abs(got["loss"]) < 4 * EPS32
    assert np.max(np.abs(got["dx"])) < 0.125 * 2 * eps_p * float(np.max(np.abs(widen(xs, "bf16"))))
    e = torch.empty((1, 1, 0, 64), dtype=torch.bfloat16, device="cuda")
    loss, dx = gpu_lib.loss(e, e)
    torch.cuda.synchronize()
    assert float(loss.cpu()) == 0.0 and dx.numel() == 0


def test_growing_logits_exercise_online_rescaling(gpu_lib):
    # Row norms grow along the sequence, so the running max changes at every
    # key tile and late keys dominate early ones by > 2^30.
    n, d = 320, 64
    rng = np.random.default_rng(8)
    g = np.linspace(0.3, 3.0, n)[:, None]
    xt = rng.standard_normal((1, 1, n, d)) * g
    xs = xt + 0.2 * rng.standard_normal((1, 1, n, d)) * g
    xt, xs = si.round_bf16_bits(xt), si.round_bf16_bits(xs)
    got = _run(gpu_lib, xt, xs, "bf16", 0.5)
    a, b = widen(xt, "bf16"), widen(xs, "bf16")
    ref = oracle.relation_kl(a, b, 0.5, True)
    _compare(got, ref, "bf16", n, _logit_bound(a, b, 0.5))


def test_loss_only_matches_full(gpu_lib):
    # Loss only runs the one-sweep forward path; the full path forms the KL in
    # phase 2.  Both are checked against the oracle, and against each other at
    # the per-row KL bound.
    import torch
    xt, xs = random_pair(1, 2, 190, 128, 0.3, seed=4)
    a, b = to_device(xt, "bf16"), to_device(xs, "bf16")
    s = 1.0 / np.sqrt(128)
    l1, _ = gpu_lib.loss(a, b, need_dx=False)
    l2, _ = gpu_lib.loss(a, b, need_dx=True)
    torch.cuda.synchronize()
    ref = oracle.relation_kl(widen(xt, "bf16"), widen(xs, "bf16"), f32(s), True)["loss"]
    assert rel(float(l1.cpu()), ref) < TOL["bf16"]["loss"]
    assert rel(float(l2.cpu()), ref) < TOL["bf16"]["loss"]
    zmax = _logit_bound(widen(xt, "bf16"), widen(xs, "bf16"), s)
    assert abs(float(l1.cpu()) - float(l2.cpu())) < 2 * (TOL["bf16"]["kl"] + 8 * EPS32 * zmax) * 2


def _fwd_compare(got_lt, got_ls, got_kl, ref, dtype, zmax):
    tol = TOL[dtype]
    scale_err = (EPS32 * zmax * 8) if dtype == "bf16" else 0.0
    for g, k in ((got_lt, "lse_t"), (got_ls, "lse_s")):
        err = np.max(np.abs(g - ref[k]))
        assert err < tol["lse"] * (1 + np.max(np.abs(ref[k]))) + scale_err, (k, err)
    kl_err = np.max(np.abs(got_kl - ref["row_kl"]))
    assert kl_err < tol["kl"] + 1e-4 * np.max(np.abs(ref["row_kl"])) + scale_err, kl_err


def _run_fwd(lmr, xt_np, xs_np, dtype, scale, causal=True):
    import torch
    xt, xs = to_device(xt_np, dtype), to_device(xs_np, dtype)
    lt, ls, kl = lmr.kl_fwd(xt, xs, scale, causal)
    torch.cuda.synchronize()
    return lt.cpu().numpy(), ls.cpu().numpy(), kl.cpu().numpy()


@pytest.mark.parametrize("n", [1, 2, 63, 64, 65, 129, 200, 257, 333, 513])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [True, False])
def test_kl_fwd_ragged(gpu_lib, n, d, causal):
    """Forward-only sweep: LSE and row KL in one pass against the dense oracle."""
    xt, xs = random_pair(1, 2, n, d, 0.4, seed=n * 3 + d + causal)
    s = 1.0 / np.sqrt(d)
    a, b = widen(xt, "bf16"), widen(xs, "bf16")
    ref = oracle.relation_kl(a, b, f32(s), causal)
    _fwd_compare(*_run_fwd(gpu_lib, xt, xs, "bf16", s, causal), ref, "bf16", _logit_bound(a, b, s))


@pytest.mark.parametrize("n", [1, 100, 257])
def test_kl_fwd_fp32(gpu_lib, n):
    xt, xs = random_pair(2, 1, n, 64, 0.4, seed=40 + n, dtype="f32")
    s = 1.0 / 8.0
    a, b = widen(xt, "f32"), widen(xs, "f32")
    ref = oracle.relation_kl(a, b, f32(s), True)
    _fwd_compare(*_run_fwd(gpu_lib, xt, xs, "f32", s), ref, "f32", _logit_bound(a, b, s))


def test_kl_fwd_identical_inputs_give_exact_zero(gpu_lib):
    xt, _ = random_pair(1, 3, 260, 128, 0.0, seed=13)
    lt, ls, kl = _run_fwd(gpu_lib, xt, xt.copy(), "bf16", 1 / np.sqrt(128))
    assert np.all(kl == 0.0) and np.array_equal(lt, ls)


@pytest.mark.parametrize("causal", [True, False])
def test_kl_fwd_overflowing_shift_takes_the_exact_fallback(gpu_lib, causal):
    n, d = 150, 64
    rng = np.random.default_rng(12)
    xt = rng.standard_normal((1, 2, n, d))
    xt[:, :, 3] *= 30.0
    xs = xt + 0.3 * rng.standard_normal((1, 2, n, d))
    xt, xs = si.round_bf16_bits(xt), si.round_bf16_bits(xs)
    got = _run_fwd(gpu_lib, xt, xs, "bf16", 0.125, causal)
    a, b = widen(xt, "bf16"), widen(xs, "bf16")
    ref = oracle.relation_kl(a, b, 0.125, causal)
    assert all(np.all(np.isfinite(g)) for g in got)
    _fwd_compare(*got, ref, "bf16", _logit_bound(a, b, 0.125))


def test_kl_fwd_peaky_heads(gpu_lib):
    # Per-head projection scales as in the GQA workload: some rows put almost
    # all probability on the diagonal.
    w = si.workload("llama3_gqa_8k", n=384, B=1)
    m = si.make_inputs(w, maps=["K"])["K"]
    a, b = m.xt64[:, :4], m.xs64[:, :4]
    got = _run_fwd(gpu_lib, np.ascontiguousarray(m.xt[:, :4]), np.ascontiguousarray(m.xs[:, :4]), "bf16", w.scale)
    ref = oracle.relation_kl(a, b, f32(w.scale), True)
    _fwd_compare(*got, ref, "bf16", _logit_bound(a, b, w.scale))


@pytest.mark.parametrize("mode", MODES)
def test_phase2_modes_are_bitwise_deterministic(gpu_lib, mode):
    import torch
    xt, xs = random_pair(1, 4, 700, 128, 0.3, seed=6)
    a, b = to_device(xt, "bf16"), to_device(xs, "bf16")
    outs = []
    for _ in range(3):
        loss, dx = gpu_lib.loss(a, b, dx_mode=mode)
        torch.cuda.synchronize()
        outs.append((float(loss.cpu()), dx.cpu().numpy()))
    for o in outs[1:]:
        assert o[0] == outs[0][0] and np.array_equal(o[1], outs[0][1])


@pytest.mark.parametrize("causal", [True, False])
def test_fused_and_split_agree(gpu_lib, causal):
    """The two phase-2 modes add the same terms in different orders: the row KL
    and loss are bit for bit the same (same row sweep arithmetic), the gradient
    agrees to fp32 rounding."""
    import torch
    xt, xs = random_pair(2, 3, 611, 128, 0.3, seed=21)
    a, b = to_device(xt, "bf16"), to_device(xs, "bf16")
    lt, ls = gpu_lib.lse_fwd(a, b, None, causal)
    kf, df = gpu_lib.kl_bwd(a, b, lt, ls, None, causal, dx_mode=gpu_lib.DX_FUSED)
    ks, ds = gpu_lib.kl_bwd(a, b, lt, ls, None, causal, dx_mode=gpu_lib.DX_SPLIT)
    torch.cuda.synchronize()
    assert torch.equal(kf, ks)
    e = float((df - ds).abs().max() / ds.abs().max())
    print(f"  fused vs split (causal={causal}): normwise max difference {e:.2e}", flush=True)
    assert e < 1e-5


@pytest.mark.parametrize("causal", [True, False])
def test_overflowing_shift_takes_the_exact_fallback(gpu_lib, causal):
    # Row 3 has a huge norm, so for the rows after it a logit exceeds the
    # row's own diagonal logit by far more than fp32 exp2 can represent;
    # phase 1 must fall back to the online maximum and stay exact.
    n, d = 150, 64
    rng = np.random.default_rng(12)
    xt = rng.standard_normal((1, 2, n, d))
    xt[:, :, 3] *= 30.0
    xs = xt + 0.3 * rng.standard_normal((1, 2, n, d))
    xt, xs = si.round_bf16_bits(xt), si.round_bf16_bits(xs)
    got = _run(gpu_lib, xt, xs, "bf16", 0.125, causal=causal)
    a, b = widen(xt, "bf16"), widen(xs, "bf16")
    ref = oracle.relation_kl(a, b, 0.125, causal)
    assert np.all(np.isfinite(got["lse_t"])) and np.all(np.isfinite(got["dx"]))
    _compare(got, ref, "bf16", n, _logit_bound(a, b, 0.125))


# Phase 1 switches to its wide shape (12 waves, 384-row blocks, 96-row key
# tiles) when that grid has at least 1024 workgroups.  Many heads at ragged
# lengths reach it at small n; sampled heads are checked against the oracle.
WIDE_GRID = 1024


def _wide_heads(n):
    """Head count (B = 2) whose wide phase-1 grid reaches WIDE_GRID."""
    blocks = -(-n // 384)
    return -(-WIDE_GRID // (2 * blocks))


@pytest.mark.parametrize("n,d", [(385, 128), (500, 64), (777, 128), (1152, 128)])
def test_wide_phase1_shape(gpu_lib, n, d):
    import torch
    H = _wide_heads(n)
    xt, xs = random_pair(2, H, n, d, 0.4, seed=n + d)
    s = 1.0 / np.sqrt(d)
    a, b = to_device(xt, "bf16"), to_device(xs, "bf16")
    ws = torch.empty(gpu_lib.workspace_bytes(2, H, n), dtype=torch.uint8, device="cuda")
    loss, dx = gpu_lib.loss(a, b, s, True, workspace=ws)
    f_lt, f_ls, f_kl = gpu_lib.kl_fwd(a, b, s, True)
    torch.cuda.synchronize()
    off = gpu_lib.workspace_layout(2, H, n)
    lse_t = ws[off[0]:off[0] + 8 * 2 * H * n].view(torch.float64).view(2, H, n).cpu().numpy()
    row_kl = ws[off[2]:off[2] + 4 * 2 * H * n].view(torch.float32).view(2, H, n).cpu().numpy()
    # Every row's sum runs over the same 32-row blocks in the same order in
    # either phase-1 shape, so the forward-only sweep's LSE is bit-equal.
    assert np.array_equal(f_lt.cpu().numpy(), lse_t)
    rng = np.random.default_rng(n)
    for bb, hh in [(0, 0), (1, H - 1), (int(rng.integers(2)), int(rng.integers(H)))]:
        xa, xb = widen(xt[bb, hh], "bf16"), widen(xs[bb, hh], "bf16")
        ref = oracle.relation_kl_head(xa, xb, f32(s), True)
        zmax = _logit_bound(xa, xb, s)
        assert np.max(np.abs(lse_t[bb, hh] - ref["lse_t"])) < 2e-6 * (1 + np.max(np.abs(ref["lse_t"]))) + 8 * EPS32 * zmax
        kl_tol = 2e-6 + 1e-4 * np.max(np.abs(ref["row_kl"])) + 8 * EPS32 * zmax
        assert np.max(np.abs(row_kl[bb, hh] - ref["row_kl"])) < kl_tol
        assert np.max(np.abs(f_kl[bb, hh].cpu().numpy() - ref["row_kl"])) < kl_tol
        assert normwise_max_rel(dx[bb, hh].cpu().numpy(), ref["dself"]) < 2e-2


@pytest.mark.parametrize("causal", [True, False])
def test_wide_phase1_overflow_fallback(gpu_lib, causal):
    """Huge-norm rows in some heads make the fixed shift overflow: those 384-row
    blocks of the wide phase 1 redo their rows with the online maximum."""
    import torch
    n, d = 450, 64
    H = _wide_heads(n)
    rng = np.random.default_rng(21)
    xt = rng.standard_normal((2, H, n, d))
    xt[:, ::37, 3] *= 30.0
    xt[:, ::53, 400] *= 30.0
    xs = xt + 0.3 * rng.standard_normal(xt.shape)
    xt, xs = si.round_bf16_bits(xt), si.round_bf16_bits(xs)
    a, b = to_device(xt, "bf16"), to_device(xs, "bf16")
    lt, ls = gpu_lib.lse_fwd(a, b, 0.125, causal)
    f_lt, f_ls, f_kl = gpu_lib.kl_fwd(a, b, 0.125, causal)
    torch.cuda.synchronize()
    # (The forward-only sweep keeps 256-row blocks, so its fallback re-sums
    # other sets of rows with the online maximum: both exact, not bit-equal.)
    for bb, hh in [(0, 0), (1, 37), (0, 53), (1, 106)]:
        xa, xb = widen(xt[bb, hh], "bf16"), widen(xs[bb, hh], "bf16")
        ref = oracle.relation_kl_head(xa, xb, 0.125, causal)
        zmax = _logit_bound(xa, xb, 0.125)
        for got, want in ((lt, ref["lse_t"]), (ls, ref["lse_s"]), (f_lt, ref["lse_t"]), (f_ls, ref["lse_s"])):
            g = got[bb, hh].cpu().numpy()
            assert np.all(np.isfinite(g))
            assert np.max(np.abs(g - want)) < 2e-6 * (1 + np.max(np.abs(want))) + 8 * EPS32 * zmax
        kl_tol = 2e-6 + 1e-4 * np.max(np.abs(ref["row_kl"])) + 8 * EPS32 * zmax
        assert np.max(np.abs(f_kl[bb, hh].cpu().numpy() - ref["row_kl"])) < kl_tol


@pytest.mark.parametrize("n,expect", [(8192, 3), (8193, 1)])
def test_auto_mode_choice(gpu_lib, n, expect):
    """AUTO runs the fused phase 2 up to n = 8192 and the split sweeps above:
    its gradient equals that mode's bit for bit (the two modes differ in the
    last bits)."""
    import torch
    xt, xs = random_pair(1, 1, n, 64, 0.3, seed=n)
    a, b = to_device(xt, "bf16"), to_device(xs, "bf16")
    _, d_auto = gpu_lib.loss(a, b, dx_mode=gpu_lib.DX_AUTO)
    _, d_want = gpu_lib.loss(a, b, dx_mode=expect)
    _, d_other = gpu_lib.loss(a, b, dx_mode=4 - expect if expect == 3 else 3)
    torch.cuda.synchronize()
    assert torch.equal(d_auto, d_want)
    assert not torch.equal(d_auto, d_other)


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("B,H", [(1, 64), (3, 24)])
def test_head_groups_match_one_launch(gpu_lib, mode, B, H):
    """larard_loss runs phase 1 per head group and phase 2 per sub-group
    (n = 8448, d = 128: groups of 62 heads of the flattened B*H, sub-groups of
    32; with B = 3, H = 24 the boundaries fall inside batches); its loss and
    gradient equal those of the phase entry points launched once over all
    heads, bit for bit."""
    import torch
    n, d = 8448, 128
    assert gpu_lib.loss_head_group(B, H, n, d) == 62 and gpu_lib.loss_sweep_group(B, H, n, d) == 32
    xt, xs = random_pair(B, H, n, d, 0.3, seed=21)
    a, b = to_device(xt, "bf16"), to_device(xs, "bf16")
    s = 1.0 / np.sqrt(d)
    loss_g, dx_g = gpu_lib.loss(a, b, s, True, 0.5, dx_mode=mode)
    lse_t = torch.empty((B, H, n), dtype=torch.float64, device="cuda")
    lse_s = torch.empty_like(lse_t)
    gpu_lib.lse_fwd(a, b, s, True, lse_t, lse_s)
    row_kl, dx1 = gpu_lib.kl_bwd(a, b, lse_t, lse_s, s, True, 0.5, dx_mode=mode)
    partials = torch.empty((B * H,), dtype=torch.float64, device="cuda")
    loss1 = torch.empty((), dtype=torch.float32, device="cuda")
    gpu_lib.reduce_loss(row_kl, partials, loss1, 0.5)
    torch.cuda.synchronize()
    assert torch.equal(dx_g, dx1)
    assert float(loss_g.cpu()) == float(loss1.cpu())
