"""Pins for the fp64 CPU oracle, none of which reuses the oracle's own formulas.

* exact worked examples (tests/golden, rational arithmetic from the definition);
* torch's fp64 CPU scaled_dot_product_attention and its autograd (a library routine
  and automatic differentiation, versus the oracle's hand-derived backward);
* a numpy brute force with plain exp/sum and no max subtraction;
* central finite differences of L = sum(O * dO), element-wise and along the gradient
  and a random direction, at the awkward sizes of the page "A transformer in PTX",
  section "Checking the gradients" (head size 12, 4 query heads over 2 key/value
  heads, 3 sequences of 9 tokens);
* closed forms and invariants: row 0, Q = 0 (prefix means, LSE = ln(i+1)),
  rows of P summing to one, the null space of the softmax gradient, invariance under a
  shift of K, GQA equal to MHA with repeated K/V, independence of batches.
"""
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import synthetic_inputs as si

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
AWKWARD = dict(B=3, T=9, Hq=4, Hkv=2, d=12)


def f64_inputs(B, T, Hq, Hkv, d, seed, qk_mult=1.0):
    x = si.make_inputs(B, T, Hq, Hkv, d, seed, qk_mult)
    return {n: si.bf16_bits_to_f32(a).astype(np.float64) for n, a in x.items()}


# ----------------------------------------------------------------------------- golden
def _read_golden(name):
    vals = {}
    shape = None
    scale_txt = None
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            parts = line.split()
            if parts[0] == "shape":
                shape = {kv.split("=")[0]: int(kv.split("=")[1]) for kv in parts[1:]}
                continue
            if parts[0] == "scale":
                scale_txt = parts[1]
                continue
            vals.setdefault(parts[0], []).append(parts[1:])
    B, T, Hq, Hkv, d = (shape[k] for k in ("B", "T", "Hq", "Hkv", "d"))

    def arr(key, H):
        a = np.zeros((1, T, H, d))
        for row in vals[key]:
            t, h = int(row[0]), int(row[1])
            a[0, t, h] = [float(Fraction(x)) for x in row[2:]]
        return a

    lse_exp = np.zeros((1, Hq, T))
    for row in vals["lse_exp"]:
        lse_exp[0, int(row[0])] = [float(Fraction(x)) for x in row[1:]]
    scale = math.log(2.0) if scale_txt == "ln2" else float(Fraction(scale_txt))
    return dict(q=arr("q", Hq), k=arr("k", Hkv), v=arr("v", Hkv), do=arr("do", Hq),
                o=arr("o", Hq), lse=np.log(lse_exp), dq=scale * arr("dq_over_scale", Hq),
                dk=scale * arr("dk_over_scale", Hkv), dv=arr("dv", Hkv), scale=scale)


@pytest.mark.parametrize("name", ["pow2_scores.txt", "uniform_scores.txt"])
def test_golden_worked_examples(oracle_mod, name):
    g = _read_golden(name)
    r = oracle_mod.attn_bwd(g["q"], g["k"], g["v"], g["do"], g["scale"])
    for key in ("o", "lse", "dq", "dk", "dv"):
        np.testing.assert_allclose(r[key], g[key], rtol=1e-12, atol=1e-12, err_msg=key)
    fo, flse = oracle_mod.attn_fwd(g["q"], g["k"], g["v"], g["scale"])
    np.testing.assert_allclose(fo, g["o"], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(flse, g["lse"], rtol=1e-12, atol=1e-12)


# ------------------------------------------------------------------ torch library pin
def _torch_ref(x, scale):
    """fp64 CPU: torch SDPA (causal, GQA by repeating K/V) and autograd."""
    G = x["q"].shape[2] // x["k"].shape[2]
    q = torch.tensor(x["q"]).permute(0, 2, 1, 3).requires_grad_(True)   # [B,H,T,d]
    k = torch.tensor(x["k"]).permute(0, 2, 1, 3).requires_grad_(True)
    v = torch.tensor(x["v"]).permute(0, 2, 1, 3).requires_grad_(True)
    kr = k.repeat_interleave(G, dim=1)
    vr = v.repeat_interleave(G, dim=1)
    o = torch.nn.functional.scaled_dot_product_attention(q, kr, vr, is_causal=True, scale=scale)
    T = q.shape[2]
    mask = torch.ones(T, T, dtype=torch.bool).tril()
    s = (q @ kr.transpose(-1, -2)) * scale
    lse = torch.logsumexp(s.masked_fill(~mask, float("-inf")), dim=-1)
    do = torch.tensor(x["do"]).permute(0, 2, 1, 3)
    (o * do).sum().backward()
    perm = lambda t: t.detach().permute(0, 2, 1, 3).numpy()
    return dict(o=perm(o), lse=lse.detach().numpy(), dq=perm(q.grad), dk=perm(k.grad),
                dv=perm(v.grad))


@pytest.mark.parametrize("shape,seed,mult", [
    (AWKWARD, 1, 1.0),
    (dict(B=1, T=64, Hq=6, Hkv=2, d=64), 2, 1.0),
    (dict(B=2, T=33, Hq=4, Hkv=4, d=16), 3, 2.0),
    (dict(B=1, T=17, Hq=8, Hkv=1, d=8), 4, 1.0),
])
def test_matches_torch_sdpa_and_autograd(oracle_mod, shape, seed, mult):
    x = f64_inputs(**shape, seed=seed, qk_mult=mult)
    scale = 1.0 / math.sqrt(shape["d"])
    r = oracle_mod.attn_bwd(x["q"], x["k"], x["v"], x["do"], scale)
    ref = _torch_ref(x, scale)
    for key in ("o", "lse", "dq", "dk", "dv"):
        np.testing.assert_allclose(r[key], ref[key], rtol=1e-10, atol=1e-11, err_msg=key)


# ---------------------------------------------------------------- numpy brute force
def _brute_fwd(x, scale):
    q, k, v = x["q"], x["k"], x["v"]
    B, T, Hq, d = q.shape
    G = Hq // k.shape[2]
    o = np.zeros_like(q)
    lse = np.zeros((B, Hq, T))
    for b in range(B):
        for h in range(Hq):
            s = scale * q[b, :, h] @ k[b, :, h // G].T
            e = np.where(np.tril(np.ones((T, T), bool)), np.exp(s), 0.0)
            z = e.sum(axis=1)
            o[b, :, h] = (e / z[:, None]) @ v[b, :, h // G]
            lse[b, h] = np.log(z)
    return o, lse


@pytest.mark.parametrize("shape,seed", [(AWKWARD, 5), (dict(B=1, T=64, Hq=6, Hkv=2, d=64), 1)])
def test_matches_brute_force(oracle_mod, shape, seed):
    x = f64_inputs(**shape, seed=seed)
    scale = 1.0 / math.sqrt(shape["d"])
    o, lse = oracle_mod.attn_fwd(x["q"], x["k"], x["v"], scale)
    bo, blse = _brute_fwd(x, scale)
    np.testing.assert_allclose(o, bo, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse, blse, rtol=1e-12, atol=1e-13)


# ------------------------------------------------------------- finite differences
def _loss(oracle_mod, x, scale):
    o, _ = oracle_mod.attn_fwd(x["q"], x["k"], x["v"], scale, threads=1)
    return float(np.sum(o * x["do"]))


def test_finite_differences_elementwise(oracle_mod):
    shape = dict(B=1, T=5, Hq=4, Hkv=2, d=3)
    x = f64_inputs(**shape, seed=9)
    scale = 0.7
    r = oracle_mod.attn_bwd(x["q"], x["k"], x["v"], x["do"], scale)
    eps = 1e-6
    for name, gname in (("q", "dq"), ("k", "dk"), ("v", "dv")):
        g = r[gname]
        fd = np.zeros_like(g)
        for idx in np.ndindex(g.shape):
            xp = {n: a.copy() for n, a in x.items()}
            xm = {n: a.copy() for n, a in x.items()}
            xp[name][idx] += eps
            xm[name][idx] -= eps
            fd[idx] = (_loss(oracle_mod, xp, scale) - _loss(oracle_mod, xm, scale)) / (2 * eps)
        np.testing.assert_allclose(g, fd, rtol=1e-6, atol=1e-8, err_msg=gname)


@pytest.mark.parametrize("direction", ["gradient", "random"])
def test_finite_differences_directional(oracle_mod, direction):
    x = f64_inputs(**AWKWARD, seed=12)
    scale = 1.0 / math.sqrt(AWKWARD["d"])
    r = oracle_mod.attn_bwd(x["q"], x["k"], x["v"], x["do"], scale)
    rng = np.random.default_rng(99)
    for name, gname in (("q", "dq"), ("k", "dk"), ("v", "dv")):
        g = r[gname]
        u = g.copy() if direction == "gradient" else rng.standard_normal(g.shape)
        u /= np.linalg.norm(u)
        eps = 1e-5
        xp = dict(x); xp[name] = x[name] + eps * u
        xm = dict(x); xm[name] = x[name] - eps * u
        fd = (_loss(oracle_mod, xp, scale) - _loss(oracle_mod, xm, scale)) / (2 * eps)
        gu = float(np.sum(g * u))
        assert abs(fd - gu) <= 1e-7 * max(1.0, abs(gu)), (name, fd, gu)


# ---------------------------------------------------------- closed forms, invariants
def test_row_zero_closed_form(oracle_mod):
    x = f64_inputs(2, 7, 6, 3, 16, seed=4)
    scale = 0.25
    o, lse = oracle_mod.attn_fwd(x["q"], x["k"], x["v"], scale)
    for b in range(2):
        for h in range(6):
            g = h // 2
            np.testing.assert_array_equal(o[b, 0, h], x["v"][b, 0, g])
            want = scale * math.fsum(x["q"][b, 0, h] * x["k"][b, 0, g])
            assert abs(lse[b, h, 0] - want) <= 1e-14 * max(1, abs(want))


def test_lse_identity_fsum(oracle_mod):
    x = f64_inputs(1, 12, 2, 1, 8, seed=6, qk_mult=2.0)
    scale = 0.35
    _, lse = oracle_mod.attn_fwd(x["q"], x["k"], x["v"], scale)
    for h in range(2):
        for i in range(12):
            s = [scale * math.fsum(x["q"][0, i, h] * x["k"][0, j, 0]) for j in range(i + 1)]
            want = math.log(math.fsum(math.exp(t) for t in s))
            assert abs(lse[0, h, i] - want) <= 1e-13 * max(1, abs(want))


def test_zero_queries_prefix_mean(oracle_mod):
    B, T, Hq, Hkv, d = 2, 40, 6, 2, 8
    x = f64_inputs(B, T, Hq, Hkv, d, seed=8)
    x["q"][:] = 0.0
    r = oracle_mod.attn_bwd(x["q"], x["k"], x["v"], x["do"], 0.125)
    cnt = np.arange(1, T + 1, dtype=np.float64)
    for b in range(B):
        for h in range(Hq):
            g = h // 3
            prefix = np.cumsum(x["v"][b, :, g], axis=0) / cnt[:, None]
            np.testing.assert_allclose(r["o"][b, :, h], prefix, rtol=1e-12, atol=1e-13)
            np.testing.assert_allclose(r["lse"][b, h], np.log(cnt), rtol=0, atol=1e-13)
    assert np.all(r["dk"] == 0.0)
    for b in range(B):
        for g in range(Hkv):
            w = x["do"][b, :, 3 * g:3 * g + 3].sum(axis=1) / cnt[:, None]   # sum_h dO_i/(i+1)
            want = np.cumsum(w[::-1], axis=0)[::-1]                          # sum over i >= j
            np.testing.assert_allclose(r["dv"][b, :, g], want, rtol=1e-12, atol=1e-12)


def test_probability_rows_sum_to_one(oracle_mod):
    x = f64_inputs(1, 30, 4, 2, 16, seed=10, qk_mult=2.0)
    c = np.linspace(-3, 3, 16)
    x["v"][:] = c
    o, _ = oracle_mod.attn_fwd(x["q"], x["k"], x["v"], 0.25)
    np.testing.assert_allclose(o, np.broadcast_to(c, o.shape), rtol=0, atol=1e-14)


def test_gradient_null_space(oracle_mod):
    x = f64_inputs(2, 50, 6, 2, 16, seed=13)
    r = oracle_mod.attn_bwd(x["q"], x["k"], x["v"], x["do"], 0.25)
    # sum_j dS_ij = 0 for every row, so the column sums of dK vanish;
    # the rows of P sum to one, so the column sums of dV equal those of dO per group.
    np.testing.assert_allclose(r["dk"].sum(axis=1), 0.0, atol=1e-11)
    for g in range(2):
        want = x["do"][:, :, 3 * g:3 * g + 3].sum(axis=(1, 2))
        np.testing.assert_allclose(r["dv"][:, :, g].sum(axis=1), want, rtol=1e-12, atol=1e-11)
    # D_i = sum_j P_ij dP_ij is the same number as dO_i . O_i: checked through dQ's
    # invariance below and through the torch pin; here the delta output equals dO.O.
    np.testing.assert_allclose(r["delta"], np.einsum("bthc,bthc->bht", x["do"], r["o"]),
                               rtol=1e-13, atol=1e-13)


def test_key_shift_invariance(oracle_mod):
    x = f64_inputs(1, 20, 4, 2, 8, seed=14)
    scale = 0.3
    a = oracle_mod.attn_bwd(x["q"], x["k"], x["v"], x["do"], scale)
    c = np.linspace(-1, 1, 8)
    y = dict(x); y["k"] = x["k"] + c
    b = oracle_mod.attn_bwd(y["q"], y["k"], y["v"], y["do"], scale)
    for key in ("o", "dq", "dk", "dv"):
        np.testing.assert_allclose(a[key], b[key], rtol=1e-10, atol=1e-11, err_msg=key)
    shift = scale * np.einsum("bthc,c->bht", x["q"], c)
    np.testing.assert_allclose(b["lse"], a["lse"] + shift, rtol=1e-12, atol=1e-12)


def test_gqa_equals_mha_with_repeated_kv(oracle_mod):
    B, T, Hq, Hkv, d = 2, 16, 6, 2, 8
    x = f64_inputs(B, T, Hq, Hkv, d, seed=15)
    a = oracle_mod.attn_bwd(x["q"], x["k"], x["v"], x["do"], 0.4)
    rep = dict(x)
    rep["k"] = np.repeat(x["k"], 3, axis=2)
    rep["v"] = np.repeat(x["v"], 3, axis=2)
    m = oracle_mod.attn_bwd(rep["q"], rep["k"], rep["v"], rep["do"], 0.4)
    for key in ("o", "lse", "dq"):
        np.testing.assert_allclose(a[key], m[key], rtol=1e-13, atol=1e-14)
    for key in ("dk", "dv"):
        summed = m[key].reshape(B, T, Hkv, 3, d).sum(axis=3)
        np.testing.assert_allclose(a[key], summed, rtol=1e-12, atol=1e-13)


def test_batches_are_independent(oracle_mod):
    x = f64_inputs(3, 12, 4, 2, 8, seed=16)
    a = oracle_mod.attn_bwd(x["q"], x["k"], x["v"], x["do"], 0.5)
    perm = [2, 0, 1]
    y = {n: v[perm] for n, v in x.items()}
    b = oracle_mod.attn_bwd(y["q"], y["k"], y["v"], y["do"], 0.5)
    for key in ("o", "lse", "dq", "dk", "dv"):
        np.testing.assert_array_equal(a[key][perm], b[key])


def test_thread_count_does_not_change_bits(oracle_mod):
    x = f64_inputs(2, 33, 6, 2, 16, seed=17)
    a = oracle_mod.attn_bwd(x["q"], x["k"], x["v"], x["do"], 0.25, threads=1)
    b = oracle_mod.attn_bwd(x["q"], x["k"], x["v"], x["do"], 0.25, threads=7)
    for key in a:
        np.testing.assert_array_equal(a[key], b[key])


def test_degenerate_sizes(oracle_mod):
    # T = 1: one key only; empty batch: nothing to do.
    x = f64_inputs(2, 1, 4, 2, 8, seed=18)
    r = oracle_mod.attn_bwd(x["q"], x["k"], x["v"], x["do"], 0.5)
    np.testing.assert_array_equal(r["o"][:, 0], np.repeat(x["v"][:, 0], 2, axis=1))
    np.testing.assert_allclose(r["dq"], 0.0, atol=1e-15)
    np.testing.assert_allclose(r["dk"], 0.0, atol=1e-15)
    e = f64_inputs(0, 4, 2, 1, 8, seed=1)
    o, lse = oracle_mod.attn_fwd(e["q"], e["k"], e["v"], 0.5)
    assert o.shape == (0, 4, 2, 8) and lse.shape == (0, 2, 4)


def test_rejects_bad_arguments(oracle_mod):
    x = f64_inputs(1, 4, 3, 2, 8, seed=1)  # 3 query heads over 2 kv heads
    with pytest.raises(ValueError):
        oracle_mod.attn_fwd(x["q"], x["k"], x["v"], 0.5)
    y = f64_inputs(1, 4, 2, 1, 8, seed=1)
    with pytest.raises(ValueError):
        oracle_mod.attn_fwd(y["q"], y["k"], y["v"], -1.0)
