"""Writes the worked examples in this folder, in exact rational arithmetic.

The pages print no attention values, so these examples are worked out by hand from
the definition of causal grouped-query softmax attention and its gradient (page "A
transformer in PTX", sections "The model" and "Flash attention"), chosen so that every
quantity is exact:

* ``pow2_scores.txt``: integer Q and K with scale = ln 2, so every score is n*ln 2 with
  n an integer and exp(score) = 2**n. Softmax probabilities, O, dS, dV are rationals;
  LSE is ln of a rational; dQ and dK are ln 2 times a rational.
* ``uniform_scores.txt``: Q = 0, so every causal row of scores is zero and row i's
  probabilities are all 1/(i+1): O is a prefix mean of V and LSE_i = ln(i+1).

This script imports neither the oracle nor the HIP library; it only evaluates the
definition with ``fractions.Fraction``. Run it from the repository root:
``python tests/golden/make_golden.py``.
"""
import os
from fractions import Fraction as F

HERE = os.path.dirname(os.path.abspath(__file__))


def solve(Q, K, V, dO, G, pow2):
    """Q, dO: [T][Hq][d] ints; K, V: [T][Hkv][d] ints (batch of one).

    pow2=True: score exponent n_ij = q_i.k_j, weights 2**n. pow2=False: Q must be 0
    and the weights are all 1. Returns exact O, sum-of-weights (LSE = ln of it),
    dQ/ln2 (or dQ / scale), dK/ln2 (or dK / scale), dV."""
    T, Hq, d = len(Q), len(Q[0]), len(Q[0][0])
    Hkv = len(K[0])
    O = [[[F(0)] * d for _ in range(Hq)] for _ in range(T)]
    Z = [[F(0)] * T for _ in range(Hq)]
    dQc = [[[F(0)] * d for _ in range(Hq)] for _ in range(T)]
    dKc = [[[F(0)] * d for _ in range(Hkv)] for _ in range(T)]
    dV = [[[F(0)] * d for _ in range(Hkv)] for _ in range(T)]
    for h in range(Hq):
        g = h // G
        P = [[F(0)] * T for _ in range(T)]
        dS = [[F(0)] * T for _ in range(T)]
        for i in range(T):
            w = []
            for j in range(i + 1):
                n = sum(Q[i][h][c] * K[j][g][c] for c in range(d))
                w.append(F(2) ** n if pow2 else F(1))
            z = sum(w)
            Z[h][i] = z
            for j in range(i + 1):
                P[i][j] = w[j] / z
            for c in range(d):
                O[i][h][c] = sum(P[i][j] * V[j][g][c] for j in range(i + 1))
            D = sum(F(dO[i][h][c]) * O[i][h][c] for c in range(d))
            for j in range(i + 1):
                dp = sum(F(dO[i][h][c] * V[j][g][c]) for c in range(d))
                dS[i][j] = P[i][j] * (dp - D)
            for c in range(d):
                dQc[i][h][c] = sum(dS[i][j] * K[j][g][c] for j in range(i + 1))
        for j in range(T):
            for c in range(d):
                dV[j][g][c] += sum(P[i][j] * dO[i][h][c] for i in range(j, T))
                dKc[j][g][c] += sum(dS[i][j] * Q[i][h][c] for i in range(j, T))
    return O, Z, dQc, dKc, dV


def fmt(x):
    return f"{x.numerator}/{x.denominator}"


def write(path, title, scale_txt, Q, K, V, dO, G, pow2):
    O, Z, dQc, dKc, dV = solve(Q, K, V, dO, G, pow2)
    T, Hq, d = len(Q), len(Q[0]), len(Q[0][0])
    Hkv = len(K[0])
    lines = [f"# {title}", "# Written by tests/golden/make_golden.py (exact rational arithmetic).",
             f"shape B=1 T={T} Hq={Hq} Hkv={Hkv} d={d}", f"scale {scale_txt}"]

    def dump(name, arr, H, conv):
        for t in range(T):
            for h in range(H):
                lines.append(f"{name} {t} {h} " + " ".join(conv(x) for x in arr[t][h]))

    dump("q", Q, Hq, str)
    dump("k", K, Hkv, str)
    dump("v", V, Hkv, str)
    dump("do", dO, Hq, str)
    dump("o", O, Hq, fmt)
    for h in range(Hq):
        lines.append(f"lse_exp {h} " + " ".join(fmt(z) for z in Z[h]))
    dump("dq_over_scale", dQc, Hq, fmt)
    dump("dk_over_scale", dKc, Hkv, fmt)
    dump("dv", dV, Hkv, fmt)
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")


def main():
    # T=4, Hq=4 over Hkv=2 (G=2), d=3: small integers keep the exponents in [-6, 6].
    Q = [[[1, 0, -1], [0, 1, 1], [1, 1, 0], [-1, 0, 1]],
         [[0, -1, 1], [1, 0, 0], [0, 0, 1], [1, -1, 0]],
         [[1, 1, 1], [-1, 1, 0], [0, 1, -1], [1, 0, 1]],
         [[0, 1, 0], [1, -1, 1], [-1, -1, 0], [0, 0, -1]]]
    K = [[[1, 0, 1], [0, 1, 0]],
         [[-1, 1, 0], [1, 1, -1]],
         [[0, 1, 1], [-1, 0, 1]],
         [[1, -1, 0], [0, 1, 1]]]
    V = [[[2, -1, 0], [1, 3, -2]],
         [[0, 1, 4], [-1, 0, 2]],
         [[3, 0, -1], [2, -2, 1]],
         [[-2, 2, 1], [0, 1, 3]]]
    dO = [[[1, 0, -1], [2, 1, 0], [0, -1, 1], [1, 1, 1]],
          [[-1, 2, 0], [0, 1, -1], [1, 0, 2], [-2, 0, 1]],
          [[0, 1, 1], [1, -1, 0], [2, 0, -1], [0, 2, 0]],
          [[1, 1, 0], [-1, 0, 2], [0, 1, -2], [1, -1, 1]]]
    write(os.path.join(HERE, "pow2_scores.txt"),
          "Worked example: integer Q.K with scale ln 2, so exp(score) is a power of two.",
          "ln2", Q, K, V, dO, 2, True)
    Q0 = [[[0] * 3 for _ in range(4)] for _ in range(4)]
    write(os.path.join(HERE, "uniform_scores.txt"),
          "Worked example: Q = 0, every causal score row is uniform.",
          "1/8", Q0, K, V, dO, 2, False)


if __name__ == "__main__":
    main()
