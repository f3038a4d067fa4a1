"""Naive attention on the GPU (the reference mode of page "A transformer in PTX", section
"Three ways to run it"): first pinned to the fp64 oracle, then used to check the flash
kernels on every element of every workload at full size, which the oracle can only
sample."""
import numpy as np
import pytest

import causal_gqa_flash_amd as cg
import synthetic_inputs as si
from parity_util import LSE_ABS, MAX_ABS, REL_L2, compare, oracle_run, to_device, workload_scale

pytestmark = pytest.mark.gpu

# (B, T, Hq, Hkv, d, seed, qk_mult): the pages' awkward gradient-check sizes (head 12,
# four query heads on two kv heads), single token, ragged tails, G = 1 .. 8, odd head
# dimensions; then sequences as long as one (batch, kv head) slice of the larger workloads
# (T = 1024 and 2048, d = 128, and a peaky softmax), so that the full-size comparisons
# below rest on a naive mode pinned at those lengths too.
SHAPES = [(3, 9, 4, 2, 12, 41, 1.0), (1, 1, 6, 2, 64, 42, 1.0), (2, 33, 6, 2, 64, 43, 1.0),
          (1, 100, 8, 2, 128, 44, 1.0), (2, 65, 3, 1, 32, 45, 1.0), (1, 130, 8, 1, 96, 46, 1.0),
          (1, 77, 8, 8, 64, 47, 1.0), (1, 1024, 6, 2, 64, 49, 1.0), (1, 2048, 3, 1, 64, 50, 2.0),
          (1, 1024, 4, 1, 128, 51, 1.0)]


def _naive(x, scale, B, T, Hq, Hkv, d):
    import torch
    dev = to_device(x)
    ws = torch.empty((cg.attn_naive_workspace_bytes(B, T, Hq) // 4,), dtype=torch.float32, device="cuda")
    o, lse = cg.attn_naive_fwd(dev["q"], dev["k"], dev["v"], scale=scale, workspace=ws)
    delta, dq, dk, dv = cg.attn_naive_bwd(dev["q"], dev["k"], dev["v"], dev["do"], scale=scale, workspace=ws)
    torch.cuda.synchronize()
    out = dict(o=o, lse=lse, delta=delta, dq=dq, dk=dk, dv=dv)
    return {n: t.float().cpu().numpy().astype(np.float64) for n, t in out.items()}, dev


# Naive against the oracle. The naive kernels compute in fp32 with sums of at most 2048
# terms here (recursive fp32 sums err by at most n * 2^-24 relative, 1.2e-4 at n = 2048 in
# the worst case and about sqrt(n) * 2^-24 typically), so they agree with fp64 well inside
# 1e-4 relative; o is then rounded to bf16, whose unit roundoff is 2^-8 (8 significant
# bits, round to nearest).
def _close(name, got, want, rel, atol):
    err = np.abs(got - want)
    bound = atol + rel * np.abs(want)
    assert np.all(err <= bound), (name, tuple(np.argwhere(err > bound)[0]), float(err.max()))


@pytest.mark.parametrize("B,T,Hq,Hkv,d,seed,mult", SHAPES)
def test_naive_matches_oracle(B, T, Hq, Hkv, d, seed, mult):
    print(f"naive vs oracle B={B} T={T} Hq={Hq} Hkv={Hkv} d={d} seed={seed} mult={mult}", flush=True)
    scale = 1.0 / np.sqrt(d)
    x = si.make_inputs(B, T, Hq, Hkv, d, seed, mult)
    got, _ = _naive(x, scale, B, T, Hq, Hkv, d)
    want = oracle_run(x, scale)
    _close("o", got["o"], want["o"], 2.0 ** -8 + 1e-5, 1e-6)
    _close("lse", got["lse"], want["lse"], 1e-6, 1e-5)
    for n in ("delta", "dq", "dk", "dv"):
        scale_n = float(np.abs(want[n]).max())
        _close(n, got[n], want[n], 1e-4, 1e-5 * scale_n + 1e-7)


def test_naive_is_repeatable():
    B, T, Hq, Hkv, d = 2, 129, 6, 2, 64
    x = si.make_inputs(B, T, Hq, Hkv, d, 48, 1.0)
    a, _ = _naive(x, 0.125, B, T, Hq, Hkv, d)
    b, _ = _naive(x, 0.125, B, T, Hq, Hkv, d)
    for n in a:
        assert np.array_equal(a[n], b[n]), n


# Flash against naive at full size, on every element. Same tolerances as against the
# oracle, except that the naive o is itself rounded to bf16 (within u |o| of the exact
# value, u = 2^-8), so o is held to MAX_ABS + u |o_naive| element-wise and REL_L2 + u in
# relative L2; delta is held to the O bound. The largest workload needs an 8.6 GB
# workspace.
BF16_U = 2.0 ** -8
@pytest.mark.parametrize("wname", [w.name for w in si.WORKLOADS])
def test_flash_matches_naive_full_size(wname):
    import torch
    w = si.WORKLOAD_BY_NAME[wname]
    x = si.make_workload_inputs(w, seed=3)
    B = w.B
    print(f"flash vs naive {wname}", flush=True)
    scale = workload_scale(w.d)
    want, dev = _naive(x, scale, B, w.T, w.Hq, w.Hkv, w.d)
    o, lse = cg.attn_fwd(dev["q"], dev["k"], dev["v"], scale=scale)
    delta, dq = cg.attn_bwd_dq(dev["q"], dev["k"], dev["v"], o, dev["do"], lse, scale=scale)
    dk, dv = cg.attn_bwd_dkv(dev["q"], dev["k"], dev["v"], dev["do"], lse, delta, scale=scale)
    torch.cuda.synchronize()
    got = {n: t.float().cpu().numpy().astype(np.float64)
           for n, t in dict(o=o, lse=lse, delta=delta, dq=dq, dk=dk, dv=dv).items()}
    msgs, ok = [], True
    for n in ("o", "lse", "delta", "dq", "dk", "dv"):
        if n == "lse":
            good, m = compare(n, got[n], want[n], rel_l2=None, max_abs=LSE_ABS)
        elif n == "o":
            err = np.abs(got[n] - want[n])
            bound = MAX_ABS + BF16_U * np.abs(want[n])
            rel = np.linalg.norm(got[n] - want[n]) / np.linalg.norm(want[n])
            good = bool(np.all(err <= bound)) and rel <= REL_L2 + BF16_U
            m = f"o: rel_l2={rel:.3e} max_abs={err.max():.3e} max err/bound={float((err / bound).max()):.3f}"
        else:
            good, m = compare(n, got[n], want[n], rel_l2=REL_L2, max_abs=MAX_ABS)
        ok &= good
        msgs.append(m)
    assert ok, "; ".join(msgs)
