"""Checks of the seeded input generator (input preparation only, no relation-KL math)."""
from fractions import Fraction

import numpy as np
import pytest

import synth_inputs as si


def test_bf16_rounding_matches_torch_for_float32_values():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(0)
    x32 = (rng.standard_normal(200000) * rng.choice([1e-3, 1.0, 50.0], 200000)).astype(np.float32)
    ours = si.round_bf16_bits(x32.astype(np.float64))
    ref = torch.from_numpy(x32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def _nearest_even_bf16(v: float) -> float:
    """Exact single rounding of a float64 to bf16 by bracketing (for normal values)."""
    f = Fraction(v)
    if f == 0:
        return 0.0
    sign = -1 if f < 0 else 1
    a = abs(f)
    e = 0
    while a >= 2:
        a /= 2; e += 1
    while a < 1:
        a *= 2; e -= 1
    q = a * 128                       # 7 fraction bits
    lo = q.numerator // q.denominator
    rem = q - lo
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and lo % 2 == 1):
        lo += 1
    return float(sign * Fraction(lo, 128) * Fraction(2) ** e)


def test_bf16_rounding_is_a_single_nearest_even_rounding():
    rng = np.random.default_rng(1)
    vals = list(rng.standard_normal(3000) * 7.0)
    # exact ties between two bf16 neighbours, and values one ulp (float64) off a tie
    for m in (1.0 + 1 / 256, 1.0 + 3 / 256, -(2.0 + 5 / 128)):
        vals += [m, np.nextafter(m, 10.0), np.nextafter(m, -10.0)]
    v = np.array(vals)
    got = si.bf16_bits_to_f64(si.round_bf16_bits(v))
    want = np.array([_nearest_even_bf16(float(t)) for t in v])
    assert np.array_equal(got, want)


def test_rope_is_a_rotation_and_relative():
    rng = np.random.default_rng(2)
    d, n = 16, 40
    p = rng.standard_normal((n, d))
    c, s = si.rope_tables(n, d, 1e4)
    x = si.apply_rope(p, c, s)
    assert np.allclose(np.linalg.norm(x, axis=1), np.linalg.norm(p, axis=1), rtol=1e-14)
    # <RoPE(a, i), RoPE(b, j)> depends only on i - j
    a, b = rng.standard_normal(d), rng.standard_normal(d)
    xa = si.apply_rope(np.tile(a, (n, 1)), c, s)
    xb = si.apply_rope(np.tile(b, (n, 1)), c, s)
    dots = [xa[i] @ xb[i - 3] for i in range(3, n)]
    assert np.allclose(dots, dots[0], rtol=1e-12)


def test_seeded_and_deterministic():
    w = si.workload("llama2_4k", n=64, heads={"Q": 2, "K": 2, "V": 2})
    a = si.make_inputs(w)
    b = si.make_inputs(w)
    for k in "QKV":
        assert np.array_equal(a[k].xt, b[k].xt) and np.array_equal(a[k].xs, b[k].xs)
    # a map's values do not depend on which maps were requested
    only_v = si.make_inputs(w, maps=["V"])
    assert np.array_equal(only_v["V"].xs, a["V"].xs)


def test_unit_interpolation_gives_identical_teacher_and_student():
    w = si.workload("llama2_4k", n=96, heads={"Q": 1, "K": 1, "V": 1}, factor=1.0)
    m = si.make_inputs(w)
    assert np.array_equal(m["Q"].xt, m["Q"].xs)
    assert np.array_equal(m["K"].xt, m["K"].xs)


def test_shapes_dtypes_and_value_noise():
    w = si.workload("llama3_gqa_8k", n=128)
    m = si.make_inputs(w)
    assert m["Q"].xt.shape == (2, 32, 128, 128) and m["Q"].xt.dtype == np.uint16
    assert m["K"].xt.shape == (2, 8, 128, 128)
    dv = m["V"].xs64 - m["V"].xt64
    assert 0.045 < dv.std() < 0.055
    t = si.make_inputs(si.WORKLOADS["tiny_f32"])["Q"]
    assert t.xt.dtype == np.float32 and t.xt.shape == (1, 1, 256, 64)
    # teacher diagonal logit equals the student's up to float rounding (RoPE is a rotation)
    nt = np.sum(t.xt64[0, 0] ** 2, axis=1)
    ns = np.sum(t.xs64[0, 0] ** 2, axis=1)
    assert np.allclose(nt, ns, rtol=1e-5)
