"""Pins of the RoPE oracle (oracle/rope.py): a hand-worked rotation, the identity and
quarter turns, the transposed rotation undoing the rotation, pair norms, and the
property that makes it a position embedding: the dot product of a rotated query and a
rotated key depends only on their distance."""
import numpy as np

import synthetic_inputs as si
from oracle import rope


def test_worked_example_by_hand():
    # One token, one head, d = 4: pair 0 turns by 90 degrees, pair 1 by 0.
    x = np.array([1.0, 2.0, 3.0, 4.0]).reshape(1, 1, 1, 4)
    cos = np.array([[0.0, 1.0]])
    sin = np.array([[1.0, 0.0]])
    # pair 0: (1*0 - 2*1, 1*1 + 2*0) = (-2, 1); pair 1 unchanged.
    assert rope.rotate(x, cos, sin).ravel().tolist() == [-2.0, 1.0, 3.0, 4.0]
    assert rope.rotate_back(rope.rotate(x, cos, sin), cos, sin).ravel().tolist() == [1.0, 2.0, 3.0, 4.0]


def test_identity_and_transpose():
    rng = np.random.default_rng(21)
    x = rng.standard_normal((2, 9, 3, 12))
    zero_c, zero_s = np.ones((9, 6)), np.zeros((9, 6))
    assert np.array_equal(rope.rotate(x, zero_c, zero_s), x)
    cos, sin = si.rope_tables(9, 12)
    y = rope.rotate(x, cos, sin)
    assert np.allclose(rope.rotate_back(y, cos, sin), x, atol=1e-6)   # tables are fp32-rounded
    # each pair keeps its length (up to the fp32 rounding of the table)
    n0 = x[..., 0::2] ** 2 + x[..., 1::2] ** 2
    n1 = y[..., 0::2] ** 2 + y[..., 1::2] ** 2
    assert np.allclose(n0, n1, rtol=1e-6)


def test_relative_position_property():
    # (R_t q) . (R_s k) = q^T R_{s-t} k depends on s - t only: shifting both positions
    # by the same amount leaves every dot product unchanged.
    rng = np.random.default_rng(22)
    d, T = 16, 40
    cos, sin = si.rope_tables(T, d)
    q = rng.standard_normal(d)
    k = rng.standard_normal(d)
    def dot(t, s):
        qs = np.zeros((1, T, 1, d)); qs[0, t, 0] = q
        ks = np.zeros((1, T, 1, d)); ks[0, s, 0] = k
        return float(rope.rotate(qs, cos, sin)[0, t, 0] @ rope.rotate(ks, cos, sin)[0, s, 0])
    for t, s, shift in [(3, 1, 10), (7, 7, 20), (2, 9, 25), (0, 5, 33)]:
        assert abs(dot(t, s) - dot(t + shift, s + shift)) < 1e-5


def test_tables_match_their_definition():
    cos, sin = si.rope_tables(5, 8, base=100.0)
    # pair 1 of token 3: angle 3 * 100^(-2/8) = 3 / sqrt(10)
    ang = 3 * 100.0 ** (-0.25)
    assert abs(cos[3, 1] - np.cos(ang)) < 1e-7 and abs(sin[3, 1] - np.sin(ang)) < 1e-7
    assert np.all(cos[0] == 1.0) and np.all(sin[0] == 0.0)


def test_rotate_bf16_rounds_the_rotated_value():
    rng = np.random.default_rng(23)
    x = si.f32_to_bf16_bits(rng.standard_normal((1, 6, 2, 8), dtype=np.float32))
    cos, sin = si.rope_tables(6, 8)
    r = rope.rotate_bf16(x, cos, sin)
    exact = rope.rotate(si.bf16_bits_to_f32(x).astype(np.float64), cos, sin)
    # bf16 values within half a unit (2^-8 relative) of the exact rotation
    assert np.all(np.abs(r - exact) <= 2.0 ** -8 * np.abs(exact) + 1e-30)
    # and every value is a bf16 number (widening its bits gives it back)
    assert np.array_equal(si.bf16_bits_to_f32(si.f32_to_bf16_bits(r.astype(np.float32))), r.astype(np.float32))


def test_fma32_is_the_exact_value_rounded_once():
    from fractions import Fraction
    rng = np.random.default_rng(24)
    a = rng.standard_normal(3000).astype(np.float32)
    b = rng.standard_normal(3000).astype(np.float32)
    c = (rng.standard_normal(3000) * 10.0 ** rng.integers(-8, 3, 3000)).astype(np.float32)
    # constructed halfway cases: a*b lands exactly between two float32 numbers next to c
    for i in range(0, 200):
        c[i] = np.float32(1.0)
        a[i] = np.float32(1.0)
        b[i] = np.float32(2.0 ** -24 * (1 + 2 * (i % 2)))   # 1 + 2^-24 (tie) or 1 + 3 * 2^-24
    got = rope.fma32(a, b, c)

    def round32(fr):
        # nearest float32 to a Fraction (ties to even), by bracketing with nextafter
        f = np.float32(float(fr))
        lo, hi = (f, np.nextafter(f, np.float32(np.inf))) if Fraction(float(f)) <= fr else \
                 (np.nextafter(f, np.float32(-np.inf)), f)
        dlo, dhi = fr - Fraction(float(lo)), Fraction(float(hi)) - fr
        if dlo < dhi:
            return lo
        if dhi < dlo:
            return hi
        return lo if (int(np.float32(lo).view(np.uint32)) & 1) == 0 else hi

    for i in range(len(a)):
        exact = Fraction(float(a[i])) * Fraction(float(b[i])) + Fraction(float(c[i]))
        assert got[i] == round32(exact), (i, a[i], b[i], c[i], got[i])


def test_fp32_rotation_rounds_like_the_exact_one_almost_always():
    rng = np.random.default_rng(25)
    x = si.f32_to_bf16_bits(rng.standard_normal((2, 64, 3, 64), dtype=np.float32))
    cos, sin = si.rope_tables(64, 64)
    a = rope.rotate_bf16_fp32(x, cos, sin)
    b = rope.rotate_bf16(x, cos, sin)
    ulp = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(b), 1e-30))) - 7)
    assert np.all(np.abs(a - b) <= ulp)
    assert np.mean(a == b) > 0.99
