"""Several maps in one launch per phase (larard_multi_loss) against per-map calls and the oracle.

The fused kernels run the same per-head arithmetic as the per-map launches,
only scheduled together, so each map's gradient must match the per-map path
bit for bit (weights are powers of two, so the gradient scale rounds the
same way); the loss is the weighted sum, reduced in fp64.  Both the loss and
every map's fused gradient are also compared with the fp64 oracle.
"""
import numpy as np
import pytest

import oracle
import synth_inputs as si
from helpers import normwise_max_rel, rel, to_device, widen

pytestmark = pytest.mark.gpu


def _maps_gqa(B, n, d, Hs, seed, dtype="bf16"):
    rng = np.random.default_rng(seed)
    out = []
    for H in Hs:
        xt = rng.standard_normal((B, H, n, d)) * rng.uniform(0.5, 1.5, (1, H, 1, 1))
        xs = xt + 0.3 * rng.standard_normal(xt.shape)
        rnd = si.round_bf16_bits if dtype == "bf16" else si.round_f32
        out.append((rnd(xt), rnd(xs)))
    return out


@pytest.mark.parametrize("n,d,causal", [(200, 128, True), (129, 64, True), (150, 128, False), (1, 128, True),
                                         (300, 128, True)])
def test_multi_matches_per_map_and_oracle(gpu_lib, n, d, causal):
    import torch
    Hs, weights = (4, 2, 2), (1.0, 0.5, 2.0)
    host = _maps_gqa(2, n, d, Hs, seed=n + d)
    dev = [(to_device(a, "bf16"), to_device(b, "bf16")) for a, b in host]
    s = 1.0 / np.sqrt(d)
    dxs = [torch.empty(a.shape, dtype=torch.float32, device="cuda") for a, _ in dev]
    loss = gpu_lib.multi_loss([(a, b, w, g) for (a, b), w, g in zip(dev, weights, dxs)], s, causal, 0.25)
    loss_only = gpu_lib.multi_loss([(a, b, w, None) for (a, b), w in zip(dev, weights)], s, causal, 0.25)
    singles = [gpu_lib.loss(a, b, s, causal, 0.25 * w) for (a, b), w in zip(dev, weights)]
    torch.cuda.synchronize()
    want = sum(float(l.cpu()) for l, _ in singles)
    assert rel(float(loss.cpu()), want) < 1e-6
    assert rel(float(loss_only.cpu()), want) < 1e-5 or abs(float(loss_only.cpu()) - want) < 1e-7
    for g, (_, dx1) in zip(dxs, singles):
        assert torch.equal(g, dx1)
    # and against the oracle: the weighted loss, and every map's fused bf16
    # gradient (normwise max-relative, the bf16 bar)
    refs = [oracle.relation_kl(widen(a, "bf16"), widen(b, "bf16"), float(np.float32(s)), causal, 0.25 * w)
            for (a, b), w in zip(host, weights)]
    ref = sum(r["loss"] for r in refs)
    if abs(ref) > 1e-6:
        assert rel(float(loss.cpu()), ref) < 1e-3
    for k, (g, r) in enumerate(zip(dxs, refs)):
        e = normwise_max_rel(g.cpu().numpy(), r["dxs"])
        print(f"  map {k} (H={Hs[k]}, weight {weights[k]}): fused dX normwise max-rel {e:.2e}", flush=True)
        assert e < 2e-2, (k, e)


def test_multi_fp32(gpu_lib):
    import torch
    host = _maps_gqa(1, 90, 64, (2, 1), seed=5, dtype="f32")
    dev = [(to_device(a, "f32"), to_device(b, "f32")) for a, b in host]
    dxs = [torch.empty(a.shape, dtype=torch.float32, device="cuda") for a, _ in dev]
    loss = gpu_lib.multi_loss([(a, b, 1.0, g) for (a, b), g in zip(dev, dxs)], 0.125, True)
    torch.cuda.synchronize()
    refs = [oracle.relation_kl(a.astype(np.float64), b.astype(np.float64), 0.125, True) for a, b in host]
    assert rel(float(loss.cpu()), sum(r["loss"] for r in refs)) < 1e-5
    for g, r in zip(dxs, refs):
        assert normwise_max_rel(g.cpu().numpy(), r["dxs"]) < 1e-5


def test_multi_large_maps_run_apart(gpu_lib):
    """Maps whose bf16 projections together exceed 256 MiB (here 2 x 64 heads at
    n = 8448, d = 128: 554 MB): larard_multi_loss runs them one after another,
    each as larard_loss would (head groups, split phase 2 above n = 8192).  Loss
    and gradients must equal the per-map calls bit for bit, and sampled
    gradient rows of one head per map match the oracle."""
    import torch
    B, n, d, Hs, weights = 1, 8448, 128, (64, 64), (1.0, 0.5)
    assert sum(B * H * n * d * 4 for H in Hs) > 256 << 20
    host = _maps_gqa(B, n, d, Hs, seed=9)
    dev = [(to_device(a, "bf16"), to_device(b, "bf16")) for a, b in host]
    s = 1.0 / np.sqrt(d)
    dxs = [torch.empty(a.shape, dtype=torch.float32, device="cuda") for a, _ in dev]
    loss = gpu_lib.multi_loss([(a, b, w, g) for (a, b), w, g in zip(dev, weights, dxs)], s, True)
    singles = [gpu_lib.loss(a, b, s, True, w) for (a, b), w in zip(dev, weights)]
    torch.cuda.synchronize()
    want = sum(float(l.cpu()) for l, _ in singles)
    assert rel(float(loss.cpu()), want) < 1e-6
    for g, (_, dx1) in zip(dxs, singles):
        assert torch.equal(g, dx1)
    s32 = float(np.float32(s))
    rng = np.random.default_rng(11)
    for k, ((a, b), w) in enumerate(zip(host, weights)):
        h = int(rng.integers(Hs[k]))
        a64, b64 = widen(a[0, h], "bf16"), widen(b[0, h], "bf16")
        rows = sorted(set([0, 1, 255, 256, n // 2, n - 2, n - 1] + list(rng.choice(n, 6, replace=False))))
        lt = np.concatenate([oracle.lse_rows(a64, s32, range(r, min(r + 1024, n))) for r in range(0, n, 1024)])
        ls = np.concatenate([oracle.lse_rows(b64, s32, range(r, min(r + 1024, n))) for r in range(0, n, 1024)])
        ref = w * oracle.dx_rows(a64, b64, s32, rows, lt, ls)
        e = normwise_max_rel(dxs[k][0, h].cpu().numpy()[rows], ref)
        print(f"  map {k} head {h}: dX normwise max-rel {e:.2e} (rows={len(rows)})", flush=True)
        assert e < 2e-2, (k, e)
