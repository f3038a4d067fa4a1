"""Planted mistakes in the oracle, on the CPU: each mutant is a copy of the oracle's C
source with one plausible error (a dropped term, a wrong sign, a wrong index, a
transposed operand), built with gcc into a temporary library. The pins (the exact worked
examples and the torch fp64 library pin) must reject every mutant, which shows they
are strong enough to catch that kind of mistake in the real oracle."""
import math
import os
import subprocess

import numpy as np
import pytest

import oracle
from test_oracle_pins import _read_golden, _torch_ref, f64_inputs

SRC = os.path.join(os.path.dirname(oracle.__file__), "cgqa_oracle.c")

MUTANTS = {
    # forward
    "scale_dropped": ("S[jj] = j->scale * acc;", "S[jj] = acc;"),
    "causal_exclusive": ("if (jj > i) { S[jj] = -INFINITY; continue; }",
                         "if (jj >= i && i > 0) { S[jj] = -INFINITY; continue; }"),
    "normaliser_skips_diagonal": ("for (int jj = 0; jj <= i; ++jj) sum += exp(S[jj] - m);",
                                  "for (int jj = 0; jj < i; ++jj) sum += exp(S[jj] - m);\n    if (i == 0) sum = 1.0;"),
    "lse_missing_max": ("const double lse = m + log(sum);", "const double lse = log(sum);"),
    "gqa_modulo": ("const int h = g * j->G + hh;\n    double* S", "const int h = hh * j->Hkv + g;\n    double* S"),
    "v_wrong_head": ("const double* vj = j->v + idx4(b, jj, g, 0, T, Hkv, d);\n        for (int c = 0; c < d; ++c) oi[c]",
                     "const double* vj = j->v + idx4(b, jj, 0, 0, T, Hkv, d);\n        for (int c = 0; c < d; ++c) oi[c]"),
    # backward
    "delta_sign": ("dS[jj] = P[jj] * (dp - D);", "dS[jj] = P[jj] * (dp + D);"),
    "delta_dropped": ("dS[jj] = P[jj] * (dp - D);", "dS[jj] = P[jj] * dp;"),
    "dq_scale_dropped": ("for (int c = 0; c < d; ++c) dqi[c] *= j->scale;", ""),
    "dq_uses_v": ("for (int c = 0; c < d; ++c) dqi[c] += dS[jj] * kj[c];",
                  "for (int c = 0; c < d; ++c) dqi[c] += dS[jj] * j->v[idx4(b, jj, g, c, T, Hkv, d)];"),
    "dk_transposed": ("const double ds = j->dS[((size_t)hh * T + i) * T + jj];",
                      "const double ds = j->dS[((size_t)hh * T + jj) * T + i];"),
    "dv_only_first_head": ("for (int hh = 0; hh < j->G; ++hh) {\n        const int h = g * j->G + hh;\n        for (int i = jj",
                           "for (int hh = 0; hh < 1; ++hh) {\n        const int h = g * j->G + hh;\n        for (int i = jj"),
    "dkv_skip_diagonal": ("for (int i = jj; i < T; ++i) {", "for (int i = jj + 1; i < T; ++i) {"),
    "dk_scale_dropped": ("for (int c = 0; c < d; ++c) dkj[c] *= j->scale;", ""),
}


def _build_mutant(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) >= 1, f"mutation anchor for {name} not found"
    path_c = tmp_path / f"{name}.c"
    path_so = tmp_path / f"lib{name}.so"
    path_c.write_text(src.replace(old, new, 1))
    subprocess.run(["gcc", "-O2", "-std=c99", "-pthread", "-fPIC", "-shared", str(path_c), "-o",
                    str(path_so), "-lm"], check=True)
    return oracle.load_library(str(path_so))


def _passes_pins(lib):
    for gname in ("pow2_scores.txt", "uniform_scores.txt"):
        g = _read_golden(gname)
        r = oracle.attn_bwd(g["q"], g["k"], g["v"], g["do"], g["scale"], lib=lib)
        for key in ("o", "lse", "dq", "dk", "dv"):
            if not np.allclose(r[key], g[key], rtol=1e-12, atol=1e-12):
                return False
    shape = dict(B=3, T=9, Hq=4, Hkv=2, d=12)
    x = f64_inputs(**shape, seed=1)
    scale = 1.0 / math.sqrt(12)
    r = oracle.attn_bwd(x["q"], x["k"], x["v"], x["do"], scale, lib=lib)
    ref = _torch_ref(x, scale)
    return all(np.allclose(r[k], ref[k], rtol=1e-10, atol=1e-11) for k in ref)


def test_unmutated_copy_passes(tmp_path):
    path_so = tmp_path / "libsame.so"
    subprocess.run(["gcc", "-O2", "-std=c99", "-pthread", "-fPIC", "-shared", SRC, "-o",
                    str(path_so), "-lm"], check=True)
    assert _passes_pins(oracle.load_library(str(path_so)))


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_reject_mutant(name, tmp_path):
    assert not _passes_pins(_build_mutant(name, tmp_path)), f"mutant {name} survived the pins"
