"""GPU parity of the projection backward dW = h^T R^T(dX_s) against the fp64 oracle.

The kernel rounds G = R^T dX_s (computed in fp32) once to bf16 and contracts
it with the bf16 hidden states on MFMA with fp32 accumulation.

The parity gate is the comparison with the exact fp64 definition
(oracle.proj_bwd on the unrounded dX_s): normwise max-relative < 1e-2, the
size of one bf16 rounding of G.

A second, tighter comparison (< 1e-4) is a MODEL OF THE KERNEL, not an
independent pin: `_g_bf16` reproduces the kernel's own fp32 operation order
for G and its bf16 rounding, and only the contraction is then done by the
oracle.  It checks that nothing but the accumulation order differs once the
rounding of G is taken as given; it says nothing about whether that rounding
is right, which only the 1e-2 comparison does.
"""
import numpy as np
import pytest

import oracle
import synth_inputs as si
from helpers import normwise_max_rel, to_device, widen

pytestmark = pytest.mark.gpu


def _tables32(n, d, base=1.0e4, pos_scale=8.0):
    c, s = si.rope_tables(n, d, base, pos_scale)
    return si.round_f32(c[:, : d // 2]), si.round_f32(s[:, : d // 2])


def _g_bf16(dx32, c32, s32):
    """G = R^T dX in fp32 in the kernel's operation order, rounded once to bf16
    (fp64 image): g1 = fma(y1, c, fp32(y2 s)), g2 = fma(y2, c, -fp32(y1 s)).  The
    fma is exact in fp64 (an fp32 product is exact there) up to the final fp32
    rounding."""
    if c32 is None:
        g = dx32.astype(np.float32)
    else:
        half = dx32.shape[-1] // 2
        y1 = dx32[..., :half].astype(np.float64)
        y2 = dx32[..., half:].astype(np.float64)
        c64, s64 = c32.astype(np.float64), s32.astype(np.float64)
        t1 = si.round_f32(y2 * s64).astype(np.float64)
        t2 = si.round_f32(y1 * s64).astype(np.float64)
        g = np.concatenate([si.round_f32(y1 * c64 + t1), si.round_f32(y2 * c64 - t2)], axis=-1)
    return si.bf16_bits_to_f64(si.round_bf16_bits(g.astype(np.float64)))


@pytest.mark.parametrize("B,n,dm,H,d,rope", [(2, 100, 256, 2, 128, True), (1, 64, 128, 2, 64, True),
                                             (3, 37, 384, 1, 128, False), (1, 300, 256, 4, 64, True)])
def test_proj_bwd_small(gpu_lib, B, n, dm, H, d, rope):
    import torch
    rng = np.random.default_rng(B * 1000 + n + dm + H + d)
    h = si.round_bf16_bits(rng.standard_normal((B, n, dm)))
    dx = si.round_f32(rng.standard_normal((B, H, n, d)) * 1e-3)
    c, s = _tables32(n, d) if rope else (None, None)
    tc = None if c is None else torch.from_numpy(c).cuda()
    ts = None if s is None else torch.from_numpy(s).cuda()
    got = gpu_lib.proj_bwd(to_device(h, "bf16").view(B, n, dm), torch.from_numpy(dx).cuda(), tc, ts)
    torch.cuda.synchronize()
    got = got.cpu().numpy()
    h64 = widen(h, "bf16")
    exact = oracle.proj_bwd(h64, dx.astype(np.float64), c, s)
    assert normwise_max_rel(got, exact) < 1e-2
    # Kernel model (not a pin): G rounded to bf16 in the kernel's own fp32
    # order, so that only the contraction's accumulation order differs.
    g = _g_bf16(dx, c, s)
    same_rounding = oracle.proj_bwd(h64, g)
    assert normwise_max_rel(got, same_rounding) < 1e-4


def test_proj_bwd_256_tiles_ragged_tokens(gpu_lib):
    """d_model = H*d = 4096 takes the 256 x 256 workgroup tile; B*n = 200
    tokens leave a ragged, zero-padded last K step."""
    test_proj_bwd_small(gpu_lib, 2, 100, 4096, 32, 128, True)


def test_proj_bwd_empty_sequence_writes_zeros(gpu_lib):
    import torch
    h = torch.empty((1, 0, 128), dtype=torch.bfloat16, device="cuda")
    dx = torch.empty((1, 1, 0, 128), dtype=torch.float32, device="cuda")
    out = torch.full((128, 128), 7.0, dtype=torch.float32, device="cuda")
    gpu_lib.proj_bwd(h, dx, out=out)
    torch.cuda.synchronize()
    assert bool((out == 0).all())


def test_projection_chain_end_to_end(gpu_lib):
    """h -> X_s = R(h W) (bf16) -> larard_loss dX_s -> larard_proj_bwd, against
    the oracle chain on the same bf16 inputs."""
    import torch
    rng = np.random.default_rng(77)
    B, n, dm, H, d = 1, 192, 256, 2, 128
    scale = 1.0 / np.sqrt(d)
    c, s = _tables32(n, d)
    h = si.round_bf16_bits(rng.standard_normal((B, n, dm)))
    W = rng.standard_normal((dm, H * d)) / np.sqrt(dm)
    h64 = widen(h, "bf16")
    proj = (h64 @ W).reshape(B, n, H, d).transpose(0, 2, 1, 3)
    xs = si.round_bf16_bits(oracle.rope_rotate(proj, c, s))
    tc, ts = si.rope_tables(n, d, 1.0e4, 1.0)
    xt = si.round_bf16_bits(oracle.rope_rotate(proj, tc[:, : d // 2], ts[:, : d // 2]))
    loss, dx = gpu_lib.loss(to_device(xt, "bf16"), to_device(xs, "bf16"), scale, True)
    dW = gpu_lib.proj_bwd(to_device(h, "bf16").view(B, n, dm), dx, torch.from_numpy(c).cuda(),
                          torch.from_numpy(s).cuda())
    torch.cuda.synchronize()
    ref_dx = oracle.relation_kl(widen(xt, "bf16"), widen(xs, "bf16"), float(np.float32(scale)), True)["dxs"]
    ref = oracle.proj_bwd(h64, ref_dx, c, s)
    assert normwise_max_rel(dW.cpu().numpy(), ref) < 2e-2
