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


def test_rotate_bf16_on_bf16_exact_cases():
    # Quarter turns and the identity move bf16 values to bf16 values: the rounding must
    # leave them alone (x = 1.5, 3.25, -0.375, 96 are bf16 numbers).
    x = si.f32_to_bf16_bits(np.array([1.5, 3.25, -0.375, 96.0], dtype=np.float32)).reshape(1, 1, 1, 4)
    cos = np.array([[0.0, 1.0]], dtype=np.float32)
    sin = np.array([[-1.0, 0.0]], dtype=np.float32)
    # pair 0 by -90 degrees: (x0*0 - x1*(-1), x0*(-1) + x1*0) = (3.25, -1.5); pair 1 kept.
    assert rope.rotate_bf16(x, cos, sin).ravel().tolist() == [3.25, -1.5, -0.375, 96.0]


def test_rotate_bf16_tie_goes_to_even():
    # x = (1 + 2^-8, 0) is not a bf16 number, but with cos = 1 the rotated value 1 + 2^-8
    # lies exactly halfway between the bf16 neighbours 1 and 1 + 2^-7: it rounds to the
    # even one, 1. And 1 + 3 * 2^-8 rounds up to 1 + 2^-6 (even).
    x64 = np.array([1.0 + 2.0 ** -8, 0.0, 1.0 + 3 * 2.0 ** -8, 0.0]).reshape(1, 1, 1, 4)
    cos = np.array([[1.0, 1.0]])
    sin = np.array([[0.0, 0.0]])
    from oracle.gemm import round_to_bf16
    assert round_to_bf16(rope.rotate(x64, cos, sin)).ravel().tolist() == [1.0, 0.0, 1.0 + 2.0 ** -6, 0.0]
