"""Rotary embedding through the C-ABI: the rotation pass against the oracle's exact
rotation rounded once to bf16 (bit for bit), in place on a packed QKV buffer, the backward's fused
transposed rotation against the plain backward, and the whole rotary forward + backward
against the fp64 oracle, on ragged shapes and the bench workload."""
import numpy as np
import pytest

import causal_gqa_flash_amd as cg
import synthetic_inputs as si
from oracle import rope as orope
from parity_util import check_all, oracle_run, to_device, workload_scale

pytestmark = pytest.mark.gpu

SHAPES = [(2, 33, 6, 2, 64, 51), (1, 130, 8, 1, 64, 52), (2, 77, 6, 2, 128, 53), (1, 257, 12, 4, 64, 54),
          (16, 1024, 6, 2, 64, 3)]


def _tables(T, d):
    import torch
    c, s = si.rope_tables(T, d)
    return c, s, torch.from_numpy(c).cuda(), torch.from_numpy(s).cuda()


def _np(t):
    return t.float().cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("B,T,Hq,Hkv,d,seed", SHAPES)
def test_rotation_pass_matches_oracle(B, T, Hq, Hkv, d, seed):
    import torch
    print(f"rope pass B={B} T={T} Hq={Hq} Hkv={Hkv} d={d}", flush=True)
    x = si.make_inputs(B, T, Hq, Hkv, d, seed, 1.0)
    c, s, dc, ds = _tables(T, d)
    dev = to_device(x)
    qr, kr = cg.rope_qk(dev["q"], dev["k"], dc, ds)
    torch.cuda.synchronize()
    for name, got, bits in (("q", qr, x["q"]), ("k", kr, x["k"])):
        # the exact rotation rounded once to bf16, element for element
        g = _np(got)
        want = orope.rotate_bf16(bits, c, s)
        bad = np.argwhere(g != want)
        assert bad.size == 0, f"{name}: {len(bad)} elements differ, first {tuple(bad[0])}"


def test_rotation_in_place_on_packed_buffer():
    import torch
    B, T, Hq, Hkv, d = 2, 100, 6, 2, 64
    x = si.make_inputs(B, T, Hq, Hkv, d, 55, 1.0)
    _, _, dc, ds = _tables(T, d)
    dev = to_device(x)
    q_ref, k_ref = cg.rope_qk(dev["q"], dev["k"], dc, ds)
    qkv = torch.empty((B, T, Hq + 2 * Hkv, d), dtype=torch.bfloat16, device="cuda")
    qkv[:, :, :Hq] = dev["q"]
    qkv[:, :, Hq:Hq + Hkv] = dev["k"]
    qkv[:, :, Hq + Hkv:] = dev["v"]
    qv, kv = qkv[:, :, :Hq], qkv[:, :, Hq:Hq + Hkv]
    cg.rope_qk(qv, kv, dc, ds, q_out=qv, k_out=kv)
    torch.cuda.synchronize()
    assert torch.equal(qv.contiguous().view(torch.int16), q_ref.view(torch.int16))
    assert torch.equal(kv.contiguous().view(torch.int16), k_ref.view(torch.int16))
    assert torch.equal(qkv[:, :, Hq + Hkv:].contiguous().view(torch.int16), dev["v"].view(torch.int16))


@pytest.mark.parametrize("B,T,Hq,Hkv,d,seed", SHAPES)
def test_backward_rotation_matches_transposed_plain_gradients(B, T, Hq, Hkv, d, seed):
    import torch
    x = si.make_inputs(B, T, Hq, Hkv, d, seed, 1.0)
    c, s, dc, ds = _tables(T, d)
    dev = to_device(x)
    scale = workload_scale(d)
    qr, kr = cg.rope_qk(dev["q"], dev["k"], dc, ds)
    o, lse = cg.attn_fwd(qr, kr, dev["v"], scale=scale)
    delta, dq = cg.attn_bwd_dq(qr, kr, dev["v"], o, dev["do"], lse, scale=scale)
    dk, dv = cg.attn_bwd_dkv(qr, kr, dev["v"], dev["do"], lse, delta, scale=scale)
    delta_r, dq_r = cg.attn_bwd_dq(qr, kr, dev["v"], o, dev["do"], lse, scale=scale, rope=(dc, ds))
    dk_r, dv_r = cg.attn_bwd_dkv(qr, kr, dev["v"], dev["do"], lse, delta_r, scale=scale, rope=(dc, ds))
    torch.cuda.synchronize()
    assert torch.equal(delta_r, delta) and torch.equal(dv_r, dv)
    for name, got, plain in (("dq", dq_r, dq), ("dk", dk_r, dk)):
        want = orope.rotate_back(_np(plain), c, s)
        # one fp32 rotation of fp32 values: within a few units of 2^-24 of the pair's size
        g = _np(got)
        bound = 4 * 2.0 ** -24 * (np.abs(_np(plain)) + np.abs(np.roll(_np(plain), 1, axis=-1))
                                  + np.abs(np.roll(_np(plain), -1, axis=-1))) + 1e-30
        assert np.all(np.abs(g - want) <= bound), name


@pytest.mark.parametrize("B,T,Hq,Hkv,d,seed", SHAPES)
def test_rotary_pipeline_matches_oracle(B, T, Hq, Hkv, d, seed):
    import torch
    print(f"rope pipeline B={B} T={T} Hq={Hq} Hkv={Hkv} d={d}", flush=True)
    x = si.make_inputs(B, T, Hq, Hkv, d, seed, 1.0)
    c, s, dc, ds = _tables(T, d)
    scale = workload_scale(d)
    dev = to_device(x)
    qr, kr = cg.rope_qk(dev["q"], dev["k"], dc, ds)
    o, lse = cg.attn_fwd(qr, kr, dev["v"], scale=scale)
    delta, dq = cg.attn_bwd_dq(qr, kr, dev["v"], o, dev["do"], lse, scale=scale, rope=(dc, ds))
    dk, dv = cg.attn_bwd_dkv(qr, kr, dev["v"], dev["do"], lse, delta, scale=scale, rope=(dc, ds))
    torch.cuda.synchronize()
    got = {n: _np(t) for n, t in dict(o=o, lse=lse, dq=dq, dk=dk, dv=dv).items()}
    # Oracle: the exact rotation rounded once to bf16 (as the pages' in-place pass stores
    # the rotated tensor), attention in fp64, dq and dk turned back by the transposed
    # rotation.
    xr = dict(x)
    xr["q"] = si.f32_to_bf16_bits(orope.rotate_bf16(x["q"], c, s).astype(np.float32))
    xr["k"] = si.f32_to_bf16_bits(orope.rotate_bf16(x["k"], c, s).astype(np.float32))
    want = oracle_run(xr, scale)
    want["dq"] = orope.rotate_back(want["dq"], c, s)
    want["dk"] = orope.rotate_back(want["dk"], c, s)
    ok, msg = check_all(got, want)
    assert ok, msg


FUSED_SHAPES = [s for s in SHAPES if s[4] == 64] + [(16, 500, 12, 4, 64, 56)]


@pytest.mark.parametrize("B,T,Hq,Hkv,d,seed", FUSED_SHAPES)
def test_fused_rotary_forward_matches_oracle(B, T, Hq, Hkv, d, seed):
    """attn_fwd_rope (q and k turned as they are loaded) against the fp64 oracle of the
    exactly rotated inputs, at the attention tolerances."""
    import torch
    print(f"fused rope forward B={B} T={T} Hq={Hq} Hkv={Hkv} d={d}", flush=True)
    x = si.make_inputs(B, T, Hq, Hkv, d, seed, 1.0)
    c, s, dc, ds = _tables(T, d)
    scale = workload_scale(d)
    dev = to_device(x)
    o, lse = cg.attn_fwd(dev["q"], dev["k"], dev["v"], scale=scale, rope=(dc, ds))
    torch.cuda.synchronize()
    xr = dict(x)
    xr["q"] = si.f32_to_bf16_bits(orope.rotate_bf16(x["q"], c, s).astype(np.float32))
    xr["k"] = si.f32_to_bf16_bits(orope.rotate_bf16(x["k"], c, s).astype(np.float32))
    want = oracle_run(xr, scale, backward=False)
    ok, msg = check_all(dict(o=_np(o), lse=_np(lse)), want, keys=("o", "lse"))
    assert ok, msg


def test_fused_rotary_forward_bits_on_a_quarter_turn():
    """With cos = 0 and sin = 1 the turn (x0, x1) -> (-x1, x0) is exact in bf16, so the
    fused forward must give the plain forward's bits on inputs turned on the host (a grid
    where the plain forward also runs the tiled kernel; T = 500 leaves a ragged tile whose
    table rows are clamped)."""
    import torch
    B, T, Hq, Hkv, d = 16, 500, 12, 4, 64
    x = si.make_inputs(B, T, Hq, Hkv, d, 57, 1.0)
    dev = to_device(x)
    cos = torch.zeros((T, d // 2), dtype=torch.float32, device="cuda")
    sin = torch.ones((T, d // 2), dtype=torch.float32, device="cuda")

    def quarter(t):
        y = torch.empty_like(t)
        y[..., 0::2] = -t[..., 1::2]
        y[..., 1::2] = t[..., 0::2]
        return y

    o, lse = cg.attn_fwd(dev["q"], dev["k"], dev["v"], scale=0.125, rope=(cos, sin))
    o2, lse2 = cg.attn_fwd(quarter(dev["q"]), quarter(dev["k"]), dev["v"], scale=0.125)
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(lse, lse2)


def test_fused_rotary_forward_bits_equal_pass_plus_forward():
    """The fused forward rounds every rotated value as the rotation pass does, so at the
    bench workload (where the plain forward runs the tiled kernel) it gives the bits of
    the pass followed by the plain forward."""
    import torch
    B, T, Hq, Hkv, d = 16, 1024, 6, 2, 64
    x = si.make_inputs(B, T, Hq, Hkv, d, 3, 1.0)
    _, _, dc, ds = _tables(T, d)
    dev = to_device(x)
    o, lse = cg.attn_fwd(dev["q"], dev["k"], dev["v"], scale=0.125, rope=(dc, ds))
    qr, kr = cg.rope_qk(dev["q"], dev["k"], dc, ds)
    o2, lse2 = cg.attn_fwd(qr, kr, dev["v"], scale=0.125)
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(lse, lse2)
