"""The backward's matrix products take dO (and dP, dS) in fp16, whose normal range is far
narrower than bf16's. The kernels multiply dO by powers of two before that rounding (per
query row in the dQ pass; per workgroup, lowered when a larger tile arrives, in the dK/dV
pass) and divide the sums back. These tests check that gradients of any dO magnitude
match the fp64 oracle at the usual tolerance, that a power-of-two factor on dO passes
through exactly, and that rows of very different magnitude keep their own accuracy."""
import numpy as np
import pytest

import synthetic_inputs as si
from parity_util import check_all, compare, gpu_run, oracle_run, workload_scale

pytestmark = pytest.mark.gpu

GRADS = ("delta", "dq", "dk", "dv")


def _log(msg):
    print(msg, flush=True)


def _scaled_rows(bits, factors):
    """bf16 bits times per-row powers of two `factors` (broadcast over the trailing
    axes); exact, which the round trip checks."""
    f = si.bf16_bits_to_f32(bits).astype(np.float64) * factors
    out = si.f32_to_bf16_bits(f.astype(np.float32))
    assert np.array_equal(si.bf16_bits_to_f32(out).astype(np.float64), f)
    return out


SHAPES = [
    # (B, T, Hq, Hkv, d, seed): the dK/dV variants with one, two, three (one and two
    # heads each) and four head slots at d = 64, and d = 128
    (2, 300, 6, 2, 64, 41),
    (1, 200, 6, 1, 64, 42),
    (1, 130, 8, 1, 64, 43),
    (2, 161, 4, 2, 64, 44),
    (1, 150, 4, 4, 64, 45),
    (2, 200, 6, 2, 128, 46),
]


@pytest.mark.parametrize("log2s", [-10, -16, -20, 8, 12])
@pytest.mark.parametrize("B,T,Hq,Hkv,d,seed", SHAPES[:1] + SHAPES[-1:])
def test_do_power_of_two_scale(B, T, Hq, Hkv, d, seed, log2s):
    """dO times 2^k: the gradients equal the unscaled run's times 2^k bit for bit, and
    the oracle's on the scaled inputs to the usual tolerance after dividing by 2^k."""
    _log(f"dO scale 2^{log2s} B={B} T={T} Hq={Hq} Hkv={Hkv} d={d}")
    x = si.make_inputs(B, T, Hq, Hkv, d, seed)
    scale = workload_scale(d)
    s = 2.0 ** log2s
    xs = dict(x, do=_scaled_rows(x["do"], s))
    base = gpu_run(x, scale)
    got = gpu_run(xs, scale)
    for n in ("o", "lse"):
        np.testing.assert_array_equal(got[n], base[n])
    for n in GRADS:
        np.testing.assert_array_equal(got[n], base[n] * s, err_msg=n)
    want = oracle_run(xs, scale)
    ok, msg = check_all({n: got[n] / s for n in GRADS}, {n: want[n] / s for n in GRADS},
                        keys=GRADS)
    assert ok, msg


@pytest.mark.parametrize("B,T,Hq,Hkv,d,seed", SHAPES)
def test_do_rows_spanning_exponents(B, T, Hq, Hkv, d, seed):
    """Every (batch, position) row of dO times its own 2^k, k uniform in [-24, 8]: dQ is
    checked row by row against the oracle, relative to each row's own size, and dK, dV
    (sums over rows of every size) on the whole tensor."""
    _log(f"dO rows 2^[-24,8] B={B} T={T} Hq={Hq} Hkv={Hkv} d={d}")
    x = si.make_inputs(B, T, Hq, Hkv, d, seed)
    k = np.random.default_rng(seed).integers(-24, 9, size=(B, T, 1, 1))
    x["do"] = _scaled_rows(x["do"], 2.0 ** k)
    scale = workload_scale(d)
    got = gpu_run(x, scale)
    want = oracle_run(x, scale)
    # dK and dV in units of the largest row factor (the tolerances hold for unit dO)
    top = float(2.0 ** k.max())
    ok, msg = check_all({n: got[n] / top for n in ("dk", "dv")},
                        {n: want[n] / top for n in ("dk", "dv")}, keys=("dk", "dv"))
    assert ok, msg
    # dQ and delta row by row, each in units of its own row's dO size (a row flushed or
    # rounded coarsely for being small next to others would fail here)
    unit = 2.0 ** k                                            # [B, T, 1, 1]
    ok, msg = compare("dq/row", got["dq"] / unit, want["dq"] / unit)
    assert ok, msg
    ok, msg = compare("delta/row", got["delta"] / unit[..., 0, 0][:, None, :],
                      want["delta"] / unit[..., 0, 0][:, None, :])
    assert ok, msg


@pytest.mark.parametrize("case", ["later_rows_2^14", "later_rows_2^20", "first_rows_zero"])
@pytest.mark.parametrize("B,T,Hq,Hkv,d,seed", SHAPES)
def test_do_later_tiles_larger(B, T, Hq, Hkv, d, seed, case):
    """dO tiles far larger than the first tile a dK/dV workgroup reads (which sets its
    starting scale): without lowering the scale their fp16 products would overflow. Also
    a zero first tile (the largest starting scale)."""
    _log(f"dO {case} B={B} T={T} Hq={Hq} Hkv={Hkv} d={d}")
    x = si.make_inputs(B, T, Hq, Hkv, d, seed)
    f = np.ones((B, T, 1, 1))
    if case == "first_rows_zero":
        f[:, :40] = 0.0
    else:
        f[:, T // 2:] = 2.0 ** int(case.split("^")[1])
    x["do"] = _scaled_rows(x["do"], f)
    scale = workload_scale(d)
    got = gpu_run(x, scale)
    want = oracle_run(x, scale)
    for n in GRADS:
        assert np.all(np.isfinite(got[n])), n
    ref = float(np.max(f))
    ok, msg = check_all({n: got[n] / ref for n in GRADS}, {n: want[n] / ref for n in GRADS},
                        keys=GRADS)
    assert ok, msg
