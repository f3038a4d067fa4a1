"""Both forward kernels against the fp64 oracle, each forced through CGQA_FWD_KERNEL:
the balanced kernel (pairs of 64-query blocks split over two waves per head, merged
through LDS; three query heads per kv head) on shapes that cover an even and an odd
number of query blocks (the middle block pairs with itself), short and long ranges on
both waves and a peaky softmax; and the
tiled kernel on a shape the launcher would give to the balanced one. The backward runs
on each forward's O and LSE, so its parity is checked too."""
import numpy as np
import pytest

import synthetic_inputs as si
from parity_util import check_all, gpu_run, oracle_run, slice_outputs, workload_scale

pytestmark = pytest.mark.gpu

SPLIT_SHAPES = [
    # (B, T, Hq, Hkv, seed, qk_mult)
    (1, 128, 3, 1, 21, 1.0),     # two query blocks: one pair, no steady steps
    (2, 192, 6, 2, 22, 1.0),     # three blocks: the middle one alone
    (1, 320, 3, 1, 23, 2.0),     # five blocks, peaky scores
    (3, 256, 12, 4, 24, 1.0),    # four blocks, several slices
    (1, 1024, 3, 1, 25, 2.0),    # sixteen blocks: long steady ranges on both waves
    (2, 704, 6, 2, 26, 1.0),     # eleven blocks
]


@pytest.mark.parametrize("B,T,Hq,Hkv,seed,mult", SPLIT_SHAPES)
def test_balanced_forward(monkeypatch, B, T, Hq, Hkv, seed, mult):
    print(f"balanced forward B={B} T={T} Hq={Hq} Hkv={Hkv} seed={seed}", flush=True)
    monkeypatch.setenv("CGQA_FWD_KERNEL", "split")
    x = si.make_inputs(B, T, Hq, Hkv, 64, seed, mult)
    scale = workload_scale(64)
    got = gpu_run(x, scale)
    want = oracle_run(x, scale)
    ok, msg = check_all(got, want, inputs=x)
    assert ok, msg


def test_tiled_forward_on_bench_shape(monkeypatch):
    print("tiled forward B16_T1024_Hq6_Hkv2_d64", flush=True)
    monkeypatch.setenv("CGQA_FWD_KERNEL", "tiled")
    w = si.WORKLOAD_BY_NAME["B16_T1024_Hq6_Hkv2_d64"]
    x = si.make_workload_inputs(w, seed=3)
    got = gpu_run(x, w.scale)
    for b, g in ((0, 1), (w.B - 1, 0)):
        xs = si.slice_group(x, w.Hq, w.Hkv, b, g)
        want = oracle_run(xs, w.scale)
        ok, msg = check_all(slice_outputs(got, w.Hq, w.Hkv, b, g), want)
        assert ok, f"slice b={b} g={g}: {msg}"


def test_balanced_forward_repeatable(monkeypatch):
    """Two balanced-kernel runs with unrelated work between them give the same bits."""
    import torch
    monkeypatch.setenv("CGQA_FWD_KERNEL", "split")
    x = si.make_inputs(2, 512, 6, 2, 64, 27, 1.0)
    a = gpu_run(x, workload_scale(64), backward=False)
    torch.randn(1 << 20, device="cuda").sum().item()
    b = gpu_run(x, workload_scale(64), backward=False)
    for k in ("o", "lse"):
        assert np.array_equal(a[k], b[k]), k
