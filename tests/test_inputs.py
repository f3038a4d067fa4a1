"""Seeded input generator: reproducibility, shapes, and bf16 round-to-nearest-even
checked against an independent implementation (torch's float32 -> bfloat16 cast)."""
import numpy as np
import pytest
import torch

import synthetic_inputs as si


def _torch_rne(x):
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def test_rne_edge_patterns_all_exponents():
    # Every upper half combined with the lower halves where rounding decides.
    upper = np.arange(1 << 16, dtype=np.uint32) << np.uint32(16)
    for low in (0x0000, 0x0001, 0x7FFF, 0x8000, 0x8001, 0xFFFF, 0x4000, 0xC000):
        bits = upper | np.uint32(low)
        x = bits.view(np.float32)
        finite = np.isfinite(x)
        ours = si.f32_to_bf16_bits(x)
        ref = _torch_rne(x)
        assert np.array_equal(ours[finite], ref[finite]), hex(low)
        # NaN stays NaN
        nan = np.isnan(x)
        assert np.all(np.isnan(si.bf16_bits_to_f32(ours[nan])))


def test_rne_random_patterns():
    rng = np.random.default_rng(7)
    bits = rng.integers(0, 1 << 32, size=1 << 22, dtype=np.uint64).astype(np.uint32)
    x = bits.view(np.float32)
    finite = np.isfinite(x)
    assert np.array_equal(si.f32_to_bf16_bits(x)[finite], _torch_rne(x)[finite])


def test_rne_ties_by_hand():
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7: goes to the even pattern (1.0).
    assert si.f32_to_bf16_bits(np.float32(1.0 + 2.0 ** -8)) == 0x3F80
    # 1 + 3*2^-8 is a tie between 1+2^-7 (odd) and 1+2^-6 (even): rounds up.
    assert si.f32_to_bf16_bits(np.float32(1.0 + 3 * 2.0 ** -8)) == 0x3F82
    assert si.f32_to_bf16_bits(np.float32(-2.0)) == 0xC000
    # the largest finite float32 rounds to infinity in bf16
    assert si.f32_to_bf16_bits(np.float32(3.4028235e38)) == 0x7F80


def test_seeded_and_shaped():
    a = si.make_inputs(2, 5, 4, 2, 8, seed=3)
    b = si.make_inputs(2, 5, 4, 2, 8, seed=3)
    c = si.make_inputs(2, 5, 4, 2, 8, seed=4)
    for name in ("q", "k", "v", "do"):
        assert np.array_equal(a[name], b[name])
        assert not np.array_equal(a[name], c[name])
        assert a[name].dtype == np.uint16
    assert a["q"].shape == (2, 5, 4, 8) and a["k"].shape == (2, 5, 2, 8)
    assert a["do"].shape == (2, 5, 4, 8)


def test_qk_multiplier_is_exact_doubling():
    a = si.make_inputs(1, 8, 2, 1, 16, seed=11)
    b = si.make_inputs(1, 8, 2, 1, 16, seed=11, qk_mult=2.0)
    for name in ("q", "k"):
        assert np.array_equal(si.bf16_bits_to_f32(b[name]), 2 * si.bf16_bits_to_f32(a[name]))
    assert np.array_equal(a["v"], b["v"]) and np.array_equal(a["do"], b["do"])


def test_normal_statistics():
    w = si.WORKLOADS[1]
    x = si.make_workload_inputs(w, seed=2, with_do=False)
    q = si.bf16_bits_to_f32(x["q"]).astype(np.float64)
    assert abs(q.mean()) < 0.01 and abs(q.std() - 1.0) < 0.01


def test_workload_table():
    names = [w.name for w in si.WORKLOADS]
    assert len(set(names)) == 5
    w = si.WORKLOAD_BY_NAME["B16_T1024_Hq6_Hkv2_d64"]
    assert (w.B, w.T, w.Hq, w.Hkv, w.d, w.G) == (16, 1024, 6, 2, 64, 3)
    assert w.scale == 0.125
    assert si.WORKLOADS[4].scale == np.float32(1 / np.sqrt(128))


def test_slice_group():
    x = si.make_inputs(2, 4, 6, 2, 8, seed=1)
    s = si.slice_group(x, 6, 2, b=1, g=1)
    assert np.array_equal(s["q"][0], x["q"][1, :, 3:6])
    assert np.array_equal(s["k"][0, :, 0], x["k"][1, :, 1])
