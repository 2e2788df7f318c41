"""C-ABI contract tests that need no GPU: exports, workspace sizing, validation.

Validation runs before any HIP call, so invalid arguments are rejected here
without a device.  No call in this file reaches a kernel launch.
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "larard.h")


@pytest.fixture(scope="module")
def lib():
    import linear_memory_relation_amd as lmr
    return lmr.load()


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\S.*?\b(larard_\w+)\s*\(", text, re.M)))


def test_every_declared_symbol_is_exported(lib):
    names = _declared()
    assert {"larard_lse_fwd", "larard_kl_bwd", "larard_loss", "larard_workspace_bytes"} <= set(names)
    for name in names:
        assert hasattr(lib, name), name


def test_version_and_status_strings(lib):
    import linear_memory_relation_amd as lmr
    assert "gfx950" in lmr.version()
    # the loaded library was built from the sources in this tree
    from linear_memory_relation_amd.build import source_id
    assert lmr.source_id() == source_id()
    for code in range(5):
        assert lib.larard_status_str(code).decode().startswith("LARARD_")


def test_workspace_is_linear_in_bhn(lib):
    import linear_memory_relation_amd as lmr
    up = lambda v: -(-v // 256) * 256
    for B, H, n in [(1, 32, 16384), (2, 8, 8192), (1, 1, 1), (3, 5, 129)]:
        rows = B * H * n
        for dt in (lmr.BF16, lmr.FP32):      # fp64 statistics for every input type
            nb = lmr.workspace_bytes(B, H, n, dt)
            off = lmr.workspace_layout(B, H, n, dt)
            assert off == [0, up(8 * rows), 2 * up(8 * rows), 2 * up(8 * rows) + up(4 * rows)]
            assert nb == off[3] + up(8 * B * H)
            assert nb <= 20 * rows + 8 * B * H + 4 * 256      # O(BHn) bound
    assert lmr.workspace_bytes(0, 1, 4) == 0
    assert lmr.workspace_bytes(1, 1, -1) == 0
    assert lmr.workspace_bytes(1, 1, 4, 5) == 0


FAKE = 1 << 20          # 16-byte aligned non-null address; never dereferenced


def _lse(lib, **kw):
    a = dict(xt=FAKE, xs=FAKE, dt=0, B=1, H=1, n=64, d=128, scale=0.1, causal=1, lt=FAKE, ls=FAKE)
    a.update(kw)
    return lib.larard_lse_fwd(a["xt"], a["xs"], a["dt"], a["B"], a["H"], a["n"], a["d"], a["scale"],
                              a["causal"], a["lt"], a["ls"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(xt=None), 1), (dict(xs=None), 1), (dict(xt=FAKE + 8), 1), (dict(B=0), 1), (dict(H=-1), 1),
    (dict(n=-1), 1), (dict(n=(1 << 24) + 1), 1), (dict(d=96), 2), (dict(d=256), 2), (dict(dt=7), 2),
    (dict(scale=float("nan")), 1), (dict(scale=float("inf")), 1), (dict(scale=0.0), 1),
    (dict(scale=-0.5), 1), (dict(lt=None), 1), (dict(ls=FAKE + 2), 1),
    (dict(dt=1, lt=FAKE + 4), 1), (dict(lt=FAKE + 4), 1),   # fp64 statistics: 8-byte alignment
    # fp32 kernels own 32 rows per workgroup: 8192 heads x 2^19 row blocks overflow the grid
    (dict(dt=1, H=1 << 13, n=1 << 24), 1), (dict(H=1 << 13, n=1 << 24), 1),
])
def test_lse_fwd_validation(lib, kw, code):
    assert _lse(lib, **kw) == code
    assert lib.larard_last_error().decode() != ""


def test_empty_sequence_is_a_noop(lib):
    # n == 0 launches nothing and touches no pointer.
    assert _lse(lib, n=0, xt=None, xs=None, lt=None, ls=None) == 0
    st = lib.larard_kl_bwd(None, None, 0, 1, 1, 0, 64, 0.1, 1, None, None, 1.0, None, None, 0, None)
    assert st == 0


def _fwd(lib, **kw):
    a = dict(xt=FAKE, xs=FAKE, dt=0, B=1, H=2, n=64, d=128, scale=0.1, causal=1, lt=FAKE, ls=FAKE, rk=FAKE)
    a.update(kw)
    return lib.larard_kl_fwd(a["xt"], a["xs"], a["dt"], a["B"], a["H"], a["n"], a["d"], a["scale"],
                             a["causal"], a["lt"], a["ls"], a["rk"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(rk=None), 1), (dict(rk=FAKE + 2), 1), (dict(lt=None), 1), (dict(ls=FAKE + 4), 1),
    (dict(xs=None), 1), (dict(d=80), 2), (dict(dt=3), 2), (dict(scale=0.0), 1), (dict(B=0), 1),
])
def test_kl_fwd_validation(lib, kw, code):
    assert _fwd(lib, **kw) == code
    assert lib.larard_last_error().decode() != ""


def test_kl_fwd_empty_sequence_is_a_noop(lib):
    assert _fwd(lib, n=0, xt=None, xs=None, lt=None, ls=None, rk=None) == 0


def _bwd(lib, **kw):
    a = dict(xt=FAKE, xs=FAKE, dt=0, B=1, H=2, n=64, d=64, scale=0.1, causal=1, lt=FAKE, ls=FAKE,
             lscale=1.0, rk=FAKE, dx=FAKE, mode=0)
    a.update(kw)
    return lib.larard_kl_bwd(a["xt"], a["xs"], a["dt"], a["B"], a["H"], a["n"], a["d"], a["scale"],
                             a["causal"], a["lt"], a["ls"], a["lscale"], a["rk"], a["dx"], a["mode"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(rk=None), 1), (dict(lt=None), 1), (dict(dx=FAKE + 4), 1), (dict(mode=9), 1),
    (dict(lscale=float("nan")), 1), (dict(d=32), 2),
])
def test_kl_bwd_validation(lib, kw, code):
    assert _bwd(lib, **kw) == code


def _loss(lib, ws=FAKE, wsb=1 << 30, **kw):
    a = dict(xt=FAKE, xs=FAKE, dt=0, B=1, H=2, n=64, d=128, scale=0.1, causal=1, lscale=1.0,
             loss=FAKE, dx=FAKE, mode=0)
    a.update(kw)
    return lib.larard_loss(a["xt"], a["xs"], a["dt"], a["B"], a["H"], a["n"], a["d"], a["scale"],
                           a["causal"], a["lscale"], ws, wsb, a["loss"], a["dx"], a["mode"], None)


def test_loss_workspace_checks(lib):
    import linear_memory_relation_amd as lmr
    need = lmr.workspace_bytes(1, 2, 64)
    assert _loss(lib, wsb=lmr.workspace_bytes(1, 2, 64, lmr.FP32) - 1, dt=1) == 3
    assert _loss(lib, wsb=need - 1) == 3
    assert _loss(lib, ws=None) == 3
    assert _loss(lib, ws=FAKE + 16) == 3          # not 256-byte aligned
    assert _loss(lib, loss=None) == 1
    assert _loss(lib, xt=None) == 1


def _xy(lib, fn, **kw):
    a = dict(xt=FAKE, xs=FAKE, yt=FAKE, ys=FAKE, dt=0, B=1, H=2, n=64, d=128, scale=0.1, causal=1,
             lt=FAKE, ls=FAKE, rk=FAKE, lscale=1.0, dx=FAKE, dy=FAKE, ws=FAKE, wsb=1 << 30, loss=FAKE)
    a.update(kw)
    head = (a["xt"], a["xs"], a["yt"], a["ys"], a["dt"], a["B"], a["H"], a["n"], a["d"], a["scale"], a["causal"])
    if fn == "lse":
        return lib.larard_xy_lse_fwd(*head, a["lt"], a["ls"], None)
    if fn == "fwd":
        return lib.larard_xy_kl_fwd(*head, a["lt"], a["ls"], a["rk"], None)
    if fn == "bwd":
        return lib.larard_xy_kl_bwd(*head, a["lt"], a["ls"], a["lscale"], a["rk"], a["dx"], a["dy"], None)
    return lib.larard_xy_loss(*head, a["lscale"], a["ws"], a["wsb"], a["loss"], a["dx"], a["dy"], None)


@pytest.mark.parametrize("fn", ["lse", "fwd", "bwd", "loss"])
@pytest.mark.parametrize("kw,code", [
    (dict(yt=None), 1), (dict(ys=None), 1), (dict(yt=FAKE + 8), 1), (dict(xt=None), 1),
    (dict(d=96), 2), (dict(dt=5), 2), (dict(scale=-1.0), 1),
])
def test_xy_validation(lib, fn, kw, code):
    assert _xy(lib, fn, **kw) == code
    assert lib.larard_last_error().decode() != ""


def test_xy_specific_checks(lib):
    assert _xy(lib, "bwd", rk=None) == 1
    assert _xy(lib, "bwd", dy=FAKE + 4) == 1
    assert _xy(lib, "fwd", rk=None) == 1
    assert _xy(lib, "loss", ws=None) == 3
    assert _xy(lib, "loss", dx=FAKE + 8) == 1
    # n == 0 launches nothing and needs no pointer but the loss scalar of *_loss
    for fn in ("lse", "fwd", "bwd"):
        assert _xy(lib, fn, n=0, xt=None, xs=None, yt=None, ys=None, lt=None, ls=None, rk=None) == 0


def _maps(lib, Hs=(32, 8, 8), dx=FAKE, weights=None):
    import linear_memory_relation_amd as lmr
    arr = (lmr.LarardMap * len(Hs))()
    for k, H in enumerate(Hs):
        w = 1.0 if weights is None else weights[k]
        arr[k] = lmr.LarardMap(FAKE, FAKE, H, w, dx if not isinstance(dx, list) else dx[k])
    return arr


def test_multi_workspace_is_the_single_layout_over_all_heads(lib):
    import linear_memory_relation_amd as lmr
    arr = _maps(lib)
    got = lib.larard_multi_workspace_bytes(0, 2, 100, arr, 3)
    assert got == lmr.workspace_bytes(1, 2 * 48, 100)
    assert lib.larard_multi_workspace_bytes(0, 2, 100, arr, 0) == 0
    assert lib.larard_multi_workspace_bytes(0, 2, 100, arr, 9) == 0
    assert lib.larard_multi_workspace_bytes(0, 2, 100, _maps(lib, Hs=(4, 0)), 2) == 0


def _multi(lib, arr, nm, **kw):
    a = dict(dt=0, B=2, n=64, d=128, scale=0.1, causal=1, lscale=1.0, ws=FAKE, wsb=1 << 30, loss=FAKE)
    a.update(kw)
    return lib.larard_multi_loss(arr, nm, a["dt"], a["B"], a["n"], a["d"], a["scale"], a["causal"], a["lscale"],
                                 a["ws"], a["wsb"], a["loss"], None)


def test_multi_loss_validation(lib):
    arr = _maps(lib)
    assert _multi(lib, arr, 0) == 1
    assert _multi(lib, arr, 9) == 1
    assert _multi(lib, None, 3) == 1
    assert _multi(lib, _maps(lib, dx=[FAKE, None, FAKE]), 3) == 1          # all or none
    assert _multi(lib, _maps(lib, weights=[1.0, float("nan"), 1.0]), 3) == 1
    assert _multi(lib, _maps(lib, dx=FAKE + 4), 3) == 1
    assert _multi(lib, arr, 3, d=96) == 2
    assert _multi(lib, arr, 3, loss=None) == 1
    assert _multi(lib, arr, 3, wsb=1024) == 3
    assert _multi(lib, arr, 3, ws=FAKE + 64) == 3
    assert lib.larard_last_error().decode() != ""


def _proj(lib, **kw):
    a = dict(h=FAKE, dx=FAKE, B=1, n=100, dm=256, H=2, d=128, c=FAKE, s=FAKE, ws=FAKE, wsb=1 << 30, dw=FAKE)
    a.update(kw)
    return lib.larard_proj_bwd(a["h"], a["dx"], a["B"], a["n"], a["dm"], a["H"], a["d"], a["c"], a["s"], a["ws"],
                               a["wsb"], a["dw"], None)


def test_proj_bwd_workspace_and_validation(lib):
    kp = (2 * 100 + 63) // 64 * 64
    up = lambda v: (v + 255) // 256 * 256
    # (R^T dX_s)^T in bf16, [H*d, kp]; small outputs read h in place
    assert lib.larard_proj_bwd_workspace_bytes(2, 100, 256, 2, 128) == up(2 * 128 * kp * 2)
    # 256 x 256 output tiles (dm = H*d = 4096): h^T [dm, kp] as well
    assert lib.larard_proj_bwd_workspace_bytes(1, 4096, 4096, 32, 128) == 2 * 4096 * 4096 * 2
    assert lib.larard_proj_bwd_workspace_bytes(2, 8192, 4096, 8, 128) == 1024 * 16384 * 2
    assert lib.larard_proj_bwd_workspace_bytes(1, 100, 200, 2, 128) == 0       # dm not a multiple of 128
    assert _proj(lib, dm=192) == 2
    assert _proj(lib, H=1, d=64) == 2                                          # H*d = 64
    assert _proj(lib, d=96) == 2
    assert _proj(lib, c=None) == 1                                             # tables come in pairs
    assert _proj(lib, h=None) == 1
    assert _proj(lib, dx=FAKE + 4) == 1
    assert _proj(lib, dw=None) == 1
    assert _proj(lib, wsb=1024) == 3
    assert _proj(lib, ws=FAKE + 16) == 3
    assert _proj(lib, B=0) == 1


@pytest.mark.parametrize("mode,code", [(0, 0), (1, 0), (3, 0), (2, 2), (4, 1), (-1, 1)])
def test_dx_mode_status(lib, mode, code):
    """AUTO, SPLIT and FUSED are accepted; ATOMIC is not built (LARARD_E_UNSUPPORTED, before any
    launch); anything else is invalid.  n == 0 keeps larard_kl_bwd from launching; larard_loss
    (which writes a zero loss with a kernel when n == 0) is called only with rejected modes."""
    st = lib.larard_kl_bwd(None, None, 0, 1, 1, 0, 64, 0.1, 1, None, None, 1.0, None, None, mode, None)
    assert st == code
    if code == 0:
        return
    assert _bwd(lib, mode=mode) == code
    assert _loss(lib, mode=mode) == code
    if code == 2:
        assert "ATOMIC" in lib.larard_last_error().decode()


def test_noalloc_validation_before_any_device_access(lib):
    """larard_loss_noalloc checks its arguments and the static scratch limit before it looks up
    the scratch address or launches anything."""
    import linear_memory_relation_amd as lmr

    def call(**kw):
        a = dict(xt=FAKE, xs=FAKE, dt=0, B=1, H=2, n=64, d=128, scale=0.1, causal=1, lscale=1.0,
                 loss=FAKE, dx=FAKE, mode=0)
        a.update(kw)
        return lib.larard_loss_noalloc(a["xt"], a["xs"], a["dt"], a["B"], a["H"], a["n"], a["d"], a["scale"],
                                       a["causal"], a["lscale"], a["loss"], a["dx"], a["mode"], None)
    assert lmr.workspace_bytes(1, 64, 65536) > lmr.NOALLOC_SCRATCH_BYTES >= lmr.workspace_bytes(1, 32, 65536)
    assert call(H=64, n=65536) == 3
    assert "scratch" in lib.larard_last_error().decode()
    assert call(loss=None) == 1
    assert call(dx=FAKE + 4) == 1
    assert call(mode=2) == 2
    assert call(d=96) == 2
    assert call(xt=None) == 1


def test_loss_head_group_sizes(lib):
    """Heads per group of the whole-path calls: 256 MiB of bf16 projections per
    group, at least 1024 sweep workgroups, at most B*H; fp32 runs as one group."""
    hg = lib.larard_loss_head_group
    hg.restype = ctypes.c_int64
    hg.argtypes = [ctypes.c_int32, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int32]
    assert hg(0, 1, 32, 16384, 128, 0) == 32          # 8 MiB per head: the whole map
    assert hg(0, 1, 32, 32768, 128, 0) == 16          # 16 MiB per head
    assert hg(0, 1, 32, 4096, 128, 0) == 32
    assert hg(0, 2, 32, 8192, 128, 0) == 64           # 4 MiB per head: all 64 heads
    assert hg(0, 1, 32, 32768, 128, 1) == 8           # cross: 32 MiB per head; 128 row blocks x 8 = 1024
    assert hg(0, 1, 32, 16384, 128, 1) == 16          # cross: 16 MiB per head
    assert hg(0, 1, 64, 65536, 128, 0) == 8           # 32 MiB per head
    assert hg(0, 1, 16, 131072, 128, 0) == 4          # 64 MiB per head: 4 heads x 512 row blocks = 2048
    assert hg(0, 1, 16, 262144, 128, 0) == 2          # 128 MiB per head: 2 heads x 1024 row blocks
    assert hg(1, 1, 32, 32768, 128, 0) == 32          # fp32 precision kernels: one group
    assert hg(0, 1, 32, 0, 128, 0) == 32
    sg = lib.larard_loss_sweep_group
    sg.restype = ctypes.c_int64
    sg.argtypes = hg.argtypes
    assert sg(0, 1, 32, 16384, 128, 0) == 16          # 128 MiB of projections per phase-2 sub-group
    assert sg(0, 1, 32, 32768, 128, 0) == 8           # 16 MiB per head; 128 row blocks x 8 = 1024
    assert sg(0, 1, 32, 4096, 128, 0) == 32
    assert sg(0, 2, 32, 8192, 128, 0) == 32           # 4 MiB per head
    assert sg(1, 1, 32, 32768, 128, 0) == 32 and sg(0, 0, 32, 16384, 128, 0) == 0
    assert hg(0, 0, 32, 16384, 128, 0) == 0 and hg(0, 1, 32, 16384, 96, 0) == 0 and hg(7, 1, 32, 16, 64, 0) == 0
