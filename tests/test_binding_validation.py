"""The Python binding rejects every malformed caller buffer before the C call.

The kernels index every output and statistics buffer by the shape of the
inputs, so a buffer of the wrong shape, dtype or layout would be read or
written out of bounds.  These checks need no GPU: the binding checks shape,
dtype and contiguity of every buffer first and the device last, so CPU
tensors with one malformed buffer are rejected naming that buffer, and CPU
tensors that are otherwise right are rejected for not being on a GPU.
"""
import pytest
import torch

import linear_memory_relation_amd as lmr

B, H, n, d = 1, 2, 40, 64


def _x(dtype=torch.bfloat16):
    return torch.zeros((B, H, n, d), dtype=dtype), torch.zeros((B, H, n, d), dtype=dtype)


def _stat(dtype=torch.float64, shape=(B, H, n)):
    return torch.zeros(shape, dtype=dtype)


def _f32(shape):
    return torch.zeros(shape, dtype=torch.float32)


def test_well_formed_cpu_tensors_are_rejected_for_the_device():
    xt, xs = _x()
    with pytest.raises(ValueError, match="GPU tensor"):
        lmr.lse_fwd(xt, xs)
    with pytest.raises(ValueError, match="GPU tensor"):
        lmr.kl_bwd(xt, xs, _stat(), _stat())
    with pytest.raises(ValueError, match="GPU tensor"):
        lmr.loss(xt, xs)


@pytest.mark.parametrize("which", ["lse_t", "lse_s"])
def test_lse_fwd_statistics(which):
    xt, xs = _x()
    bad = {which: _stat(torch.float32)}
    with pytest.raises(ValueError, match=which):
        lmr.lse_fwd(xt, xs, **bad)
    bad = {which: _stat(shape=(B, H, n + 1))}
    with pytest.raises(ValueError, match=which):
        lmr.lse_fwd(xt, xs, **bad)


def test_kl_fwd_row_kl():
    xt, xs = _x()
    with pytest.raises(ValueError, match="row_kl"):
        lmr.kl_fwd(xt, xs, row_kl=_f32((B, H, n - 1)))
    with pytest.raises(ValueError, match="row_kl"):
        lmr.kl_fwd(xt, xs, row_kl=_stat())


def test_kl_bwd_buffers():
    xt, xs = _x()
    with pytest.raises(ValueError, match="lse_t"):
        lmr.kl_bwd(xt, xs, _stat(torch.float32), _stat())
    with pytest.raises(ValueError, match="lse_s"):
        lmr.kl_bwd(xt, xs, _stat(), _stat(shape=(B, H * n)))
    with pytest.raises(ValueError, match="dx"):
        lmr.kl_bwd(xt, xs, _stat(), _stat(), dx=_f32((B, H, n, d // 2)))
    with pytest.raises(ValueError, match="dx"):
        lmr.kl_bwd(xt, xs, _stat(), _stat(), dx=_f32((B, H, d, n)).transpose(2, 3))
    with pytest.raises(ValueError, match="row_kl"):
        lmr.kl_bwd(xt, xs, _stat(), _stat(), row_kl=_stat())


def test_split_halves():
    xt, xs = _x()
    with pytest.raises(ValueError, match="row_kl is required"):
        lmr.kl_bwd_rows(xt, xs, _stat(), _stat(), None)
    with pytest.raises(ValueError, match="dx"):
        lmr.kl_bwd_rows(xt, xs, _stat(), _stat(), _f32((B, H, n)), dx=_stat(shape=(B, H, n, d)))
    with pytest.raises(ValueError, match="dx"):
        lmr.kl_bwd_cols(xt, xs, _stat(), _stat(), torch.zeros((B, H, n, d), dtype=torch.bfloat16))


def test_reduce_loss_buffers():
    with pytest.raises(ValueError, match="partials"):
        lmr.reduce_loss(_f32((B, H, n)), _stat(shape=(B * H - 1,)), _f32(()))
    with pytest.raises(ValueError, match="out"):
        lmr.reduce_loss(_f32((B, H, n)), _stat(shape=(B * H,)), _f32((1,)))
    with pytest.raises(ValueError, match="row_kl"):
        lmr.reduce_loss(_stat(), _stat(shape=(B * H,)), _f32(()))


def test_loss_buffers():
    xt, xs = _x()
    need = lmr.workspace_bytes(B, H, n)
    with pytest.raises(ValueError, match="workspace"):
        lmr.loss(xt, xs, workspace=torch.zeros(need - 1, dtype=torch.uint8))
    with pytest.raises(ValueError, match="out"):
        lmr.loss(xt, xs, out=torch.zeros((), dtype=torch.float64))
    with pytest.raises(ValueError, match="dx"):
        lmr.loss(xt, xs, dx=_f32((B, H + 1, n, d)))


def test_cross_relation_buffers():
    xt, xs = _x()
    yt, ys = _x()
    with pytest.raises(ValueError, match="lse_s"):
        lmr.xy_lse_fwd(xt, xs, yt, ys, lse_s=_stat(torch.float32))
    with pytest.raises(ValueError, match="row_kl"):
        lmr.xy_kl_fwd(xt, xs, yt, ys, row_kl=_f32((B, H)))
    with pytest.raises(ValueError, match="dy"):
        lmr.xy_kl_bwd(xt, xs, yt, ys, _stat(), _stat(), dy=_f32((B, H, n, d + 1)))
    with pytest.raises(ValueError, match="lse_t"):
        lmr.xy_kl_bwd(xt, xs, yt, ys, None, _stat())
    with pytest.raises(ValueError, match="dx"):
        lmr.xy_loss(xt, xs, yt, ys, dx=_stat(shape=(B, H, n, d)))
    with pytest.raises(ValueError, match="y_t"):
        lmr.xy_loss(xt, xs, yt[:, :1].contiguous(), ys[:, :1].contiguous())


def test_multi_map_buffers():
    q = _x()
    kv = (torch.zeros((B, 1, n, d), dtype=torch.bfloat16), torch.zeros((B, 1, n, d), dtype=torch.bfloat16))
    maps = [(q[0], q[1], 1.0, _f32((B, H, n, d))), (kv[0], kv[1], 1.0, _f32((B, H, n, d)))]
    with pytest.raises(ValueError, match="dx of map 1"):
        lmr.multi_loss(maps)
    with pytest.raises(ValueError, match="workspace"):
        lmr.multi_loss([(q[0], q[1], 1.0, None)], workspace=torch.zeros(8, dtype=torch.uint8))
    with pytest.raises(ValueError, match="empty"):
        lmr.multi_loss([])


def test_projection_buffers():
    h = torch.zeros((B, n, 128), dtype=torch.bfloat16)
    dx = _f32((B, H, n, d))
    full = _f32((n, d))                       # a full-width [n, d] cache is not the half-width table
    half = _f32((n, d // 2))
    with pytest.raises(ValueError, match="rope_cos"):
        lmr.proj_bwd(h, dx, full, full)
    with pytest.raises(ValueError, match="both"):
        lmr.proj_bwd(h, dx, half, None)
    with pytest.raises(ValueError, match="out"):
        lmr.proj_bwd(h, dx, half, half, out=_f32((128, H * d + 1)))
    with pytest.raises(ValueError, match="GPU tensor"):
        lmr.proj_bwd(h, dx, half, half)
