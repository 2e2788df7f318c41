"""larard_loss_noalloc (static device scratch) against larard_loss (caller workspace).

Both run the same kernels on the same inputs, so loss and gradient must agree
bit for bit.  Two calls in a row, the second with a smaller input, check that
the shared scratch carries nothing over from one call to the next; the
loss-only form and the empty sequence are covered too.
"""
import numpy as np
import pytest

from helpers import random_pair, to_device

pytestmark = pytest.mark.gpu


def _both(lmr, xt, xs, scale, causal, need_dx=True, loss_scale=1.0):
    import torch
    l1, d1 = lmr.loss(xt, xs, scale, causal, loss_scale, need_dx=need_dx)
    l2, d2 = lmr.loss_noalloc(xt, xs, scale, causal, loss_scale, need_dx=need_dx)
    torch.cuda.synchronize()
    return float(l1.cpu()), d1, float(l2.cpu()), d2


@pytest.mark.parametrize("causal", [True, False])
def test_noalloc_matches_workspace_path_two_calls(gpu_lib, causal):
    import torch
    shapes = [(2, 4, 700, 128), (1, 3, 257, 64)]          # the second call is smaller
    for k, (B, H, n, d) in enumerate(shapes):
        a, b = random_pair(B, H, n, d, 0.3, seed=31 + k)
        xt, xs = to_device(a, "bf16"), to_device(b, "bf16")
        scale = 1.0 / np.sqrt(d)
        l1, d1, l2, d2 = _both(gpu_lib, xt, xs, scale, causal, loss_scale=0.5)
        print(f"  call {k} {(B, H, n, d)} causal={causal}: loss {l2:.6e} (workspace path {l1:.6e})", flush=True)
        assert l1 == l2
        assert torch.equal(d1, d2)


def test_noalloc_loss_only_and_fp32(gpu_lib):
    a, b = random_pair(1, 2, 300, 64, 0.2, seed=5)
    l1, _, l2, d2 = _both(gpu_lib, to_device(a, "bf16"), to_device(b, "bf16"), 0.125, True, need_dx=False)
    assert d2 is None and l1 == l2
    a, b = random_pair(1, 2, 90, 64, 0.2, seed=6, dtype="f32")
    l1, d1, l2, d2 = _both(gpu_lib, to_device(a, "f32"), to_device(b, "f32"), 0.125, True)
    import torch
    assert l1 == l2 and torch.equal(d1, d2)


def test_noalloc_empty_sequence_and_size_limit(gpu_lib):
    import torch
    xt = torch.empty((1, 2, 0, 128), dtype=torch.bfloat16, device="cuda")
    out = torch.full((), 3.0, dtype=torch.float32, device="cuda")
    gpu_lib.loss_noalloc(xt, xt, 0.1, True, out=out, need_dx=False)
    torch.cuda.synchronize()
    assert float(out.cpu()) == 0.0
    # a shape whose scratch exceeds the static array is refused before any launch
    big = torch.empty((1, 64, 65536, 64), dtype=torch.bfloat16, device="cuda")
    assert gpu_lib.workspace_bytes(1, 64, 65536) > gpu_lib.NOALLOC_SCRATCH_BYTES
    with pytest.raises(gpu_lib.LarardError, match="scratch"):
        gpu_lib.loss_noalloc(big, big, 0.1, True, need_dx=False)
