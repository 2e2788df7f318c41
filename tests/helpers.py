"""Shared test helpers: moving seeded inputs to the GPU and error metrics."""
import numpy as np


def to_device(arr: np.ndarray, dtype: str):
    """Storage array (uint16 bf16 bits or float32) -> contiguous CUDA tensor."""
    import torch
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32))
    return t.cuda()


def normwise_max_rel(got: np.ndarray, ref: np.ndarray) -> float:
    """max|got - ref| / max|ref| (elementwise ratios blow up near zero gradients)."""
    den = float(np.max(np.abs(ref)))
    num = float(np.max(np.abs(np.asarray(got, np.float64) - ref)))
    return num / den if den > 0 else num


def rel(a: float, b: float) -> float:
    return abs(a - b) / abs(b) if b != 0 else abs(a - b)


def random_pair(B, H, n, d, noise, seed, dtype="bf16", rng_scale=1.0):
    """Plain Gaussian teacher/student pair (not a named workload) in storage form."""
    import synth_inputs as si
    rng = np.random.default_rng(seed)
    xt = rng.standard_normal((B, H, n, d)) * rng_scale
    xs = xt + noise * rng.standard_normal((B, H, n, d))
    if dtype == "bf16":
        return si.round_bf16_bits(xt), si.round_bf16_bits(xs)
    return si.round_f32(xt), si.round_f32(xs)


def widen(a: np.ndarray, dtype: str) -> np.ndarray:
    import synth_inputs as si
    return si.bf16_bits_to_f64(a) if dtype == "bf16" else a.astype(np.float64)
