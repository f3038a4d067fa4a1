"""Parity of the HIP path (through the C-ABI) with the fp64 CPU oracle, element by
element, on seeded bf16 inputs: small shapes that span several tiles and ragged tails,
every workload at full size (oracle on sampled (batch, kv head) slices, which are
independent), special inputs with closed forms, and determinism."""
import numpy as np
import pytest

import synthetic_inputs as si
from parity_util import (LSE_ABS, check_all, compare, gpu_run, oracle_run, slice_outputs,
                         to_device, workload_scale)

pytestmark = pytest.mark.gpu


def _log(msg):
    print(msg, flush=True)


SMALL = [
    # (B, T, Hq, Hkv, d, seed, qk_mult)
    (1, 64, 6, 2, 64, 1, 1.0),
    (1, 1, 6, 2, 64, 2, 1.0),
    (2, 2, 4, 1, 64, 3, 1.0),
    (1, 31, 3, 3, 64, 4, 1.0),
    (2, 33, 6, 2, 64, 5, 1.0),
    (1, 65, 4, 2, 128, 6, 1.0),
    (3, 100, 8, 2, 64, 7, 2.0),
    (1, 127, 2, 1, 128, 8, 1.0),
    (2, 129, 6, 2, 64, 9, 1.0),
    (1, 200, 8, 8, 128, 10, 2.0),
    (1, 257, 12, 4, 64, 11, 1.0),
    (2, 300, 4, 1, 128, 12, 1.0),
    (1, 1000, 6, 2, 64, 13, 1.0),
    # every dK/dV launch variant at d = 64: G = 2 (two head slots), G = 6 (three slots of
    # two heads), G = 8 (four slots of two waves, two heads each); and d = 128 with G = 3
    (2, 161, 4, 2, 64, 14, 1.0),
    (1, 96, 6, 1, 64, 15, 2.0),
    (1, 130, 8, 1, 64, 16, 1.0),
    (2, 77, 6, 2, 128, 17, 1.0),
    # B * Hkv divisible by 8 (the dQ and forward workgroups of one (batch, kv head) slice
    # grouped on one XCD) with ragged tails
    (4, 150, 6, 2, 64, 18, 1.0),
    (8, 45, 4, 2, 64, 19, 2.0),
    (2, 333, 12, 4, 64, 20, 1.0),
    # G divisible by 3 takes one key block per dK/dV workgroup on tiny grids (at most 32
    # workgroups of four blocks: every shape above) and four blocks otherwise: ragged
    # shapes just past that size run the four-block dealing with its zig-zag order
    (17, 100, 6, 2, 64, 22, 1.0),
    (12, 300, 3, 1, 64, 23, 2.0),
    # more heads per dK/dV slot: G = 4 and G = 12 (four slots of one and of three heads),
    # G = 16 (four heads per slot), G = 5 (one slot of five heads); d = 128 with T = 1
    (2, 190, 8, 2, 64, 24, 1.0),
    (1, 70, 12, 1, 64, 25, 1.0),
    (1, 100, 16, 1, 64, 26, 2.0),
    (2, 90, 5, 1, 64, 27, 1.0),
    (1, 1, 4, 2, 128, 28, 1.0),
]


@pytest.mark.parametrize("B,T,Hq,Hkv,d,seed,mult", SMALL)
def test_parity_small(B, T, Hq, Hkv, d, seed, mult):
    _log(f"parity small B={B} T={T} Hq={Hq} Hkv={Hkv} d={d} seed={seed}")
    x = si.make_inputs(B, T, Hq, Hkv, d, seed, mult)
    scale = workload_scale(d)
    got = gpu_run(x, scale)
    want = oracle_run(x, scale)
    ok, msg = check_all(got, want, keys=("o", "lse", "delta", "dq", "dk", "dv"), inputs=x)
    assert ok, msg


@pytest.mark.parametrize("w", si.WORKLOADS, ids=[w.name for w in si.WORKLOADS])
def test_parity_full_workload(w):
    """Full-size launch; the oracle checks (batch, kv head) slices spread evenly over the
    launch, first and last included: eight at d = 64, four at d = 128 (and the whole problem
    for the two smallest workloads). Slices are independent, so each is the oracle's full
    answer for its rows; they sit at different grid positions, XCDs and tile orders."""
    _log(f"parity full {w.name}")
    x = si.make_workload_inputs(w, seed=si.WORKLOADS.index(w) + 1)
    got = gpu_run(x, w.scale)
    if w.B * w.T <= 8 * 512:
        want = oracle_run(x, w.scale)
        ok, msg = check_all(got, want)
        assert ok, msg
        return
    n_slices = w.B * w.Hkv
    k = 8 if w.d == 64 else 4
    picks = sorted({round(i * (n_slices - 1) / (k - 1)) for i in range(k)})
    for p in picks:
        b, g = divmod(p, w.Hkv)
        _log(f"  slice b={b} g={g}")
        xs = si.slice_group(x, w.Hq, w.Hkv, b, g)
        want = oracle_run(xs, w.scale)
        ok, msg = check_all(slice_outputs(got, w.Hq, w.Hkv, b, g), want)
        assert ok, f"slice b={b} g={g}: {msg}"


@pytest.mark.parametrize("w", si.WORKLOADS[:4], ids=[w.name for w in si.WORKLOADS[:4]])
def test_zero_queries_closed_form(w):
    """Q = 0: every causal row is uniform, so O_i is the prefix mean of V (bf16 rounded)
    and LSE_i = ln(i + 1); checked on every element at full size."""
    _log(f"zero queries {w.name}")
    x = si.make_workload_inputs(w, seed=21, with_do=False)
    x["q"][:] = 0
    got = gpu_run(x, w.scale, backward=False)
    v = si.bf16_bits_to_f32(x["v"]).astype(np.float64)
    cnt = np.arange(1, w.T + 1, dtype=np.float64)
    prefix = np.cumsum(v, axis=1) / cnt[None, :, None, None]          # [B,T,Hkv,d]
    want_o = np.repeat(prefix, w.G, axis=2)
    ok, msg = compare("o", got["o"], want_o)
    assert ok, msg
    ok, msg = compare("lse", got["lse"], np.broadcast_to(np.log(cnt), got["lse"].shape),
                      rel_l2=None, max_abs=LSE_ABS)
    assert ok, msg


def test_constant_values_give_constant_output():
    """Rows of P sum to one: V equal to a bf16-exact constant per channel gives O equal
    to it (up to the rounding of the sum), at every position."""
    B, T, Hq, Hkv, d = 2, 700, 6, 2, 64
    x = si.make_inputs(B, T, Hq, Hkv, d, seed=30, qk_mult=2.0, with_do=False)
    c = si.f32_to_bf16_bits(np.linspace(-3, 3, d).astype(np.float32))
    x["v"][:] = c
    got = gpu_run(x, workload_scale(d), backward=False)
    want = np.broadcast_to(si.bf16_bits_to_f32(c).astype(np.float64), got["o"].shape)
    ok, msg = compare("o", got["o"], want, rel_l2=1e-3, max_abs=2e-2)
    assert ok, msg


def test_row_zero_closed_form():
    B, T, Hq, Hkv, d = 3, 130, 8, 2, 128
    x = si.make_inputs(B, T, Hq, Hkv, d, seed=31, with_do=False)
    scale = workload_scale(d)
    got = gpu_run(x, scale, backward=False)
    q = si.bf16_bits_to_f32(x["q"]).astype(np.float64)
    k = si.bf16_bits_to_f32(x["k"]).astype(np.float64)
    v = si.bf16_bits_to_f32(x["v"]).astype(np.float64)
    for h in range(Hq):
        g = h // (Hq // Hkv)
        np.testing.assert_array_equal(got["o"][:, 0, h], v[:, 0, g])     # bf16 exact
        want = scale * np.sum(q[:, 0, h] * k[:, 0, g], axis=-1)
        assert np.max(np.abs(got["lse"][:, h, 0] - want)) <= LSE_ABS


def _bits(t):
    import torch
    return t.contiguous().view(torch.uint8).cpu().numpy().copy()


@pytest.mark.parametrize("w", si.WORKLOADS, ids=[w.name for w in si.WORKLOADS])
def test_bitwise_repeatable(w):
    """Two runs of the three calls at full size, with unrelated device work in between,
    give identical bits for every output (every forward, dQ and dK/dV kernel variant the
    five workloads launch, d = 128 included)."""
    import torch
    import causal_gqa_flash_amd as cg
    _log(f"determinism {w.name}")
    x = to_device(si.make_workload_inputs(w, seed=3))
    runs = []
    for rep in range(2):
        o, lse = cg.attn_fwd(x["q"], x["k"], x["v"], scale=w.scale)
        delta, dq = cg.attn_bwd_dq(x["q"], x["k"], x["v"], o, x["do"], lse, scale=w.scale)
        dk, dv = cg.attn_bwd_dkv(x["q"], x["k"], x["v"], x["do"], lse, delta, scale=w.scale)
        torch.cuda.synchronize()
        runs.append([_bits(t) for t in (o, lse, delta, dq, dk, dv)])
        del o, lse, delta, dq, dk, dv
        junk = torch.randn(4096, 4096, device="cuda")
        (junk @ junk).sum().item()
        del junk
    for name, a, b in zip(("o", "lse", "delta", "dq", "dk", "dv"), *runs):
        assert np.array_equal(a, b), name


@pytest.mark.parametrize("variant", ["bf16_grads", "rope"])
@pytest.mark.parametrize("wname", ["B16_T1024_Hq6_Hkv2_d64", "B4_T4096_Hq32_Hkv8_d128"])
def test_bitwise_repeatable_variants(variant, wname):
    """The backward's other compiled variants repeat bit for bit too: bf16 gradients, and
    the rotary backward (dQ and dK turned back inside the kernels)."""
    import torch
    import causal_gqa_flash_amd as cg
    w = si.WORKLOAD_BY_NAME[wname]
    _log(f"determinism {variant} {w.name}")
    x = to_device(si.make_workload_inputs(w, seed=4))
    kw = {}
    if variant == "bf16_grads":
        kw["grad_dtype"] = torch.bfloat16
    else:
        c, s = si.rope_tables(w.T, w.d)
        kw["rope"] = (torch.from_numpy(c).cuda(), torch.from_numpy(s).cuda())
    o, lse = cg.attn_fwd(x["q"], x["k"], x["v"], scale=w.scale)
    runs = []
    for rep in range(2):
        delta, dq = cg.attn_bwd_dq(x["q"], x["k"], x["v"], o, x["do"], lse, scale=w.scale, **kw)
        dk, dv = cg.attn_bwd_dkv(x["q"], x["k"], x["v"], x["do"], lse, delta, scale=w.scale, **kw)
        torch.cuda.synchronize()
        runs.append([_bits(t) for t in (delta, dq, dk, dv)])
        del delta, dq, dk, dv
        junk = torch.randn(2048, 2048, device="cuda")
        (junk @ junk).sum().item()
    for name, a, b in zip(("delta", "dq", "dk", "dv"), *runs):
        assert np.array_equal(a, b), name


def test_batch_permutation_is_exact():
    """Batches are independent: permuting them permutes the outputs bit for bit."""
    B, T, Hq, Hkv, d = 4, 300, 6, 2, 64
    x = si.make_inputs(B, T, Hq, Hkv, d, seed=32)
    perm = [2, 0, 3, 1]
    y = {n: np.ascontiguousarray(a[perm]) for n, a in x.items()}
    gx = gpu_run(x, 0.125)
    gy = gpu_run(y, 0.125)
    for n in gx:
        np.testing.assert_array_equal(gx[n][perm], gy[n])


def test_work_order_does_not_change_bits():
    """The launch order of the work depends on the grid: with B * Hkv = 32 the forward and
    dQ keep each (batch, kv head) slice on one XCD and dK/dV deals its 256 workgroups'
    key blocks in zig-zag order; with B * Hkv = 33 neither holds. Every slice is computed
    the same way either way, so the first 32 batches come out bit for bit the same."""
    B, T, Hq, Hkv, d = 33, 1024, 3, 1, 64
    _log(f"work order B={B} vs {B - 1} T={T} Hq={Hq} Hkv={Hkv}")
    x = si.make_inputs(B, T, Hq, Hkv, d, seed=33)
    g33 = gpu_run(x, 0.125)
    g32 = gpu_run({n: np.ascontiguousarray(a[:B - 1]) for n, a in x.items()}, 0.125)
    for n in g33:
        np.testing.assert_array_equal(g33[n][:B - 1], g32[n], err_msg=n)


def test_empty_problems():
    import torch
    import causal_gqa_flash_amd as cg
    for B, T in ((0, 16), (2, 0)):
        q = torch.zeros((B, T, 4, 64), dtype=torch.bfloat16, device="cuda")
        k = torch.zeros((B, T, 2, 64), dtype=torch.bfloat16, device="cuda")
        o, lse = cg.attn_fwd(q, k, k)
        delta, dq = cg.attn_bwd_dq(q, k, k, o, q, lse)
        dk, dv = cg.attn_bwd_dkv(q, k, k, q, lse, delta)
        torch.cuda.synchronize()
        assert dk.shape == (B, T, 2, 64)


def test_side_stream():
    """Work enqueued on a non-default stream gives the same bits as on the default one."""
    import torch
    w = si.WORKLOADS[1]
    x = si.make_workload_inputs(w, seed=40)
    a = gpu_run(x, w.scale)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        b = gpu_run(x, w.scale, stream=s)
    for n in a:
        np.testing.assert_array_equal(a[n], b[n])
