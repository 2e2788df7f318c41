"""Host-side checks of bench.py's step schedule (no GPU): the timed step launches what
larard_loss launches -- phase 1 per head group, phase 2 per sub-group -- so its per-kernel
times and per-launch flops describe the library's own launches."""
import pytest


def _buf(B, H, n, d):
    import torch
    meta = dict(device="meta")
    return dict(name="Q", B=B, H=H, n=n, d=d,
                xt=torch.empty((B, H, n, d), dtype=torch.bfloat16, **meta),
                xs=torch.empty((B, H, n, d), dtype=torch.bfloat16, **meta),
                lse_t=torch.empty((B, H, n), dtype=torch.float64, **meta),
                lse_s=torch.empty((B, H, n), dtype=torch.float64, **meta),
                row_kl=torch.empty((B, H, n), dtype=torch.float32, **meta),
                dx=torch.empty((B, H, n, d), dtype=torch.float32, **meta))


@pytest.mark.parametrize("B,H,n,d,groups,subs", [
    (1, 32, 16384, 128, [32], [16, 16]),
    (1, 32, 32768, 128, [16, 16], [8, 8]),
    (1, 32, 4096, 128, [32], [32]),
    (2, 32, 8192, 128, [64], [32, 32]),
    (2, 8, 8192, 128, [16], [16]),
])
def test_head_groups_follow_the_library(B, H, n, d, groups, subs):
    import bench
    import linear_memory_relation_amd as lmr
    lmr.load()
    got = bench.head_groups(_buf(B, H, n, d))
    assert [g["heads"] for g in got] == groups
    assert [sg["heads"] for sg in got[0]["sub"]] == subs
    # every head exactly once, views of the flattened B*H heads
    assert sum(sg["heads"] for g in got for sg in g["sub"]) == B * H
    for g in got:
        assert tuple(g["xt"].shape) == (1, g["heads"], n, d) and tuple(g["lse_t"].shape) == (1, g["heads"], n)
        for sg in g["sub"]:
            assert tuple(sg["dx"].shape) == (1, sg["heads"], n, d)
