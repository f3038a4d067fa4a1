"""Both forward kernels against the fp64 oracle. The launcher picks by grid size: at
d = 64, grids that would not fill the chip with the tiled kernel (one workgroup per
128-query tile and head, three per CU) go to the key-split kernel (each 64-query tile's
query blocks shared by two waves, one over the even key blocks and one over the odd ones,
merged through LDS); larger ones to the tiled kernel. The shapes here drive each kernel
through its edge cases: one to three query blocks, ragged tails that put the partial key
block on a diagonal, query blocks with no odd key block, XCD grouping on and off, and a
peaky softmax that moves the lazy reference max in both halves of a block. The backward
runs on each forward's O and LSE, so its parity is checked too."""
import numpy as np
import pytest

import synthetic_inputs as si
from parity_util import check_all, gpu_run, oracle_run, to_device, workload_scale

pytestmark = pytest.mark.gpu


def _tiled_grid(B, T, Hq):
    return B * Hq * ((T + 127) // 128)


SPLIT_SHAPES = [
    # (B, T, Hq, Hkv, seed, qk_mult): key-split kernel (small grids)
    (1, 32, 3, 1, 51, 1.0),     # one block: the odd-key wave has nothing
    (1, 17, 3, 1, 52, 1.0),     # one ragged block
    (2, 64, 6, 2, 53, 1.0),     # two blocks
    (1, 65, 3, 1, 54, 2.0),     # three blocks, the last with one query
    (1, 129, 8, 2, 56, 1.0),    # five blocks, G = 4
    (2, 224, 6, 6, 57, 2.0),    # seven blocks, G = 1, peaky
    (1, 511, 4, 1, 58, 1.0),    # sixteen blocks, ragged, G = 4
    (8, 160, 6, 1, 59, 1.0),    # eight slices, XCD grouping, G = 6
    (4, 700, 6, 2, 60, 2.0),    # 22 blocks, eight slices, peaky
    (1, 1056, 3, 1, 61, 1.0),   # 33 blocks: long ranges on both halves
]
TILED_SHAPES = [
    # grids of at least 768 tiled workgroups at d = 64: tiled kernel
    (128, 100, 6, 2, 62, 1.0),  # one ragged 128-query tile per head, XCD grouping
    (97, 129, 8, 4, 63, 1.0),   # two tiles, the last with one query, no XCD grouping
    (16, 512, 12, 3, 64, 1.0),  # four tiles, G = 4
]


@pytest.mark.parametrize("B,T,Hq,Hkv,seed,mult", SPLIT_SHAPES)
def test_key_split_forward(B, T, Hq, Hkv, seed, mult):
    assert _tiled_grid(B, T, Hq) < 768
    print(f"key-split forward B={B} T={T} Hq={Hq} Hkv={Hkv} seed={seed}", flush=True)
    x = si.make_inputs(B, T, Hq, Hkv, 64, seed, mult)
    scale = workload_scale(64)
    got = gpu_run(x, scale)
    want = oracle_run(x, scale)
    ok, msg = check_all(got, want, keys=("o", "lse", "delta", "dq", "dk", "dv"))
    assert ok, msg


@pytest.mark.parametrize("B,T,Hq,Hkv,seed,mult", TILED_SHAPES)
def test_tiled_forward(B, T, Hq, Hkv, seed, mult):
    assert _tiled_grid(B, T, Hq) >= 768
    print(f"tiled forward B={B} T={T} Hq={Hq} Hkv={Hkv} seed={seed}", flush=True)
    x = si.make_inputs(B, T, Hq, Hkv, 64, seed, mult)
    scale = workload_scale(64)
    got = gpu_run(x, scale, backward=False)
    want = oracle_run(x, scale, backward=False)
    ok, msg = check_all(got, want, keys=("o", "lse"))
    assert ok, msg


def test_key_split_heads_do_not_mix():
    """Every head of a group given the same queries gives the same bits in every head."""
    import torch
    import causal_gqa_flash_amd as cg
    B, T, Hq, Hkv = 2, 300, 6, 2
    x = si.make_inputs(B, T, Hq, Hkv, 64, 65)
    for g in range(Hkv):
        for hh in range(1, 3):
            x["q"][:, :, 3 * g + hh] = x["q"][:, :, 3 * g]
    d = to_device(x)
    o, lse = cg.attn_fwd(d["q"], d["k"], d["v"], scale=0.125)
    torch.cuda.synchronize()
    o = o.float().cpu().numpy()
    lse = lse.cpu().numpy()
    for g in range(Hkv):
        for hh in range(1, 3):
            np.testing.assert_array_equal(o[:, :, 3 * g + hh], o[:, :, 3 * g])
            np.testing.assert_array_equal(lse[:, 3 * g + hh], lse[:, 3 * g])
