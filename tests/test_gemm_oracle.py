"""Pins of the matmul oracle (oracle/gemm.py) to things other than itself: a worked
example done by hand, a plain triple loop on tiny inputs for every layout, the layout
flags as pure transpositions, R as a pure addition, and bf16 rounding against torch's
cast."""
import itertools

import numpy as np
import torch

import synthetic_inputs as si
from oracle import gemm as og


def bits(x):
    """bf16 bit patterns of values that bf16 holds exactly."""
    b = si.f32_to_bf16_bits(np.asarray(x, dtype=np.float32))
    assert np.array_equal(si.bf16_bits_to_f32(b), np.asarray(x, dtype=np.float32))
    return b


def test_worked_example_by_hand():
    # A = [[1, 2, 3], [4, 5, 6]], B (stored [N][K]) = [[1, 0, -1], [2, 1, 0]]:
    # C[0][0] = 1 - 3 = -2, C[0][1] = 2 + 2 = 4, C[1][0] = 4 - 6 = -2, C[1][1] = 8 + 5 = 13.
    a = bits([[1, 2, 3], [4, 5, 6]])
    b = bits([[1, 0, -1], [2, 1, 0]])
    assert og.gemm(a, b).tolist() == [[-2.0, 4.0], [-2.0, 13.0]]
    # With R = [[0.5, 0], [0, -13]] added: [[-1.5, 4], [-2, 0]].
    r = np.array([[0.5, 0.0], [0.0, -13.0]])
    assert og.gemm(a, b, r).tolist() == [[-1.5, 4.0], [-2.0, 0.0]]
    # The same matrices stored the other way round give the same C.
    assert og.gemm(bits(np.array([[1, 2, 3], [4, 5, 6]]).T), b, a_km=True).tolist() == [[-2.0, 4.0], [-2.0, 13.0]]
    assert og.gemm(a, bits(np.array([[1, 0, -1], [2, 1, 0]]).T), b_kn=True).tolist() == [[-2.0, 4.0], [-2.0, 13.0]]


def _loop_gemm(A, B, R, M, N, K):
    C = [[0.0] * N for _ in range(M)]
    for m in range(M):
        for n in range(N):
            s = 0.0
            for k in range(K):
                s += A(m, k) * B(n, k)
            C[m][n] = s + (R[m][n] if R is not None else 0.0)
    return np.array(C)


def test_triple_loop_every_layout():
    rng = np.random.default_rng(7)
    M, N, K = 3, 4, 5
    for a_km, b_kn, with_r in itertools.product((False, True), repeat=3):
        a = si.f32_to_bf16_bits(rng.standard_normal((K, M) if a_km else (M, K), dtype=np.float32))
        b = si.f32_to_bf16_bits(rng.standard_normal((K, N) if b_kn else (N, K), dtype=np.float32))
        af, bf = si.bf16_bits_to_f32(a).astype(np.float64), si.bf16_bits_to_f32(b).astype(np.float64)
        A = (lambda m, k: af[k][m]) if a_km else (lambda m, k: af[m][k])
        B = (lambda n, k: bf[k][n]) if b_kn else (lambda n, k: bf[n][k])
        R = rng.standard_normal((M, N)) if with_r else None
        want = _loop_gemm(A, B, R, M, N, K)
        got = og.gemm(a, b, R, a_km=a_km, b_kn=b_kn)
        assert np.allclose(got, want, rtol=1e-14, atol=1e-14), (a_km, b_kn, with_r)


def test_layout_flags_are_transpositions_and_r_adds():
    rng = np.random.default_rng(8)
    M, N, K = 17, 9, 32
    a = si.f32_to_bf16_bits(rng.standard_normal((M, K), dtype=np.float32))
    b = si.f32_to_bf16_bits(rng.standard_normal((N, K), dtype=np.float32))
    base = og.gemm(a, b)
    assert np.array_equal(og.gemm(np.ascontiguousarray(a.T), b, a_km=True), base)
    assert np.array_equal(og.gemm(a, np.ascontiguousarray(b.T), b_kn=True), base)
    r = rng.standard_normal((M, N))
    assert np.array_equal(og.gemm(a, b, r), base + r)
    # Ones: every element is K.
    one = bits(np.ones((M, K)))
    assert np.array_equal(og.gemm(one, bits(np.ones((N, K)))), np.full((M, N), float(K)))
    # Identity on the right returns A.
    eye = bits(np.eye(K))
    assert np.array_equal(og.gemm(a, eye), si.bf16_bits_to_f32(a).astype(np.float64))


def test_round_to_bf16_matches_torch_cast():
    rng = np.random.default_rng(9)
    x = np.concatenate([rng.standard_normal(20000) * 10.0 ** rng.integers(-6, 6, 20000),
                        # exact ties between neighbours: 1 + (2j+1) * 2^-8 with j even and odd
                        1.0 + (2 * np.arange(64) + 1) * 2.0 ** -8, -(3.0 + (2 * np.arange(64) + 1) * 2.0 ** -7)])
    want = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).to(torch.float64).numpy()
    got = og.round_to_bf16(x.astype(np.float32).astype(np.float64))
    assert np.array_equal(got, want)


def test_abs_product_worked_example():
    # |A| |B|^T by hand for A = [[1, -2], [-3, 4]], B (stored [N][K]) = [[-1, 2], [0.5, -0.25]]:
    # row 0: |1|*|-1| + |-2|*|2| = 5, |1|*0.5 + |-2|*0.25 = 1; row 1: 3 + 8 = 11, 1.5 + 1 = 2.5.
    # (A plain product would give [[-5, 1], [11, -2.5]]: a dropped absolute value changes
    # the signs, a dropped term the sizes.)
    a = bits([[1, -2], [-3, 4]])
    b = bits([[-1, 2], [0.5, -0.25]])
    assert og.abs_product(a, b).tolist() == [[5.0, 1.0], [11.0, 2.5]]
    # stored the other way round: the same bound
    assert og.abs_product(bits(np.array([[1, -2], [-3, 4]]).T), b, a_km=True).tolist() == [[5.0, 1.0], [11.0, 2.5]]
    assert og.abs_product(a, bits(np.array([[-1, 2], [0.5, -0.25]]).T), b_kn=True).tolist() == [[5.0, 1.0], [11.0, 2.5]]
