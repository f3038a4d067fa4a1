"""fp64 CPU oracle for the projection matmul (test infrastructure; see the package header).

Page "A transformer in PTX", section "Three ways to run it": one matmul computes every
projection, C = A B^T with an optional matrix R added (the residual stream, or a gradient
accumulated across micro-batches), and takes flags for operands stored the other way
round (dx = dy W, dW = dy^T x) instead of transposing them in memory.

Definition used here: with A_m the [M][K] matrix (A as given, or its transpose when it
is stored [K][M]) and B_n the [N][K] matrix (likewise),

    C[m][n] = sum_k A_m[m][k] * B_n[n][k]  (+ R[m][n])

computed in float64 from the exact bf16 values. A product of two bf16 numbers is exact
in float64 and a sum of at most 2^20 such terms loses at most ~2^-33 relative, far below
any tolerance used against it. numpy's matmul is the one library step.
"""
import numpy as np

from . import bf16_to_f64


def operand(bits, k_major):
    """The [rows][K] float64 matrix of a bf16 operand stored [rows][K] or, if k_major,
    [K][rows]."""
    x = bf16_to_f64(np.ascontiguousarray(bits, dtype=np.uint16))
    return x.T if k_major else x


def gemm(a_bits, b_bits, r=None, a_km=False, b_kn=False):
    """C = A_m B_n^T (+ r) in float64 (see the module docstring)."""
    a = operand(a_bits, a_km)
    b = operand(b_bits, b_kn)
    if a.shape[1] != b.shape[1]:
        raise ValueError(f"inner sizes differ: {a.shape} and {b.shape}")
    c = a @ b.T
    if r is not None:
        c = c + np.asarray(r, dtype=np.float64)
    return c


def round_to_bf16(x):
    """Nearest bf16 value (ties to even) of each float64, for normal-range magnitudes:
    a bf16 keeps 8 significant bits, so x = m * 2^e with m in [0.5, 1) rounds to
    rint(m * 2^8) * 2^(e - 8), rint rounding halves to even."""
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)
    return np.ldexp(np.rint(m * 256.0), e - 8)


def abs_product(a_bits, b_bits, a_km=False, b_kn=False):
    """|A_m| |B_n|^T: the sum of the magnitudes of the terms of each C element, which
    bounds the rounding error of any order of summing them."""
    return np.abs(operand(a_bits, a_km)) @ np.abs(operand(b_bits, b_kn)).T
