"""Strided layouts through the C-ABI (the *_strided entry points, reached through the
binding's row-strided views): q, k, v read from one packed QKV buffer, o written into a
padded buffer and the gradients into one packed dQKV buffer give exactly the bits of the
contiguous calls; bf16 gradients are the fp32 ones rounded to nearest even and stay within
the fp32 tolerance widened by that rounding; columns outside a tensor's window keep their
previous contents."""
import numpy as np
import pytest

import causal_gqa_flash_amd as cg
import synthetic_inputs as si
from parity_util import MAX_ABS, REL_L2, oracle_run, workload_scale

pytestmark = pytest.mark.gpu

# (B, T, Hq, Hkv, d, seed): ragged tails, G = 3 and 4 (two dK/dV chunk layouts), d = 128
SHAPES = [(2, 33, 6, 2, 64, 31), (3, 100, 8, 2, 64, 32), (2, 129, 6, 2, 64, 33),
          (1, 257, 12, 4, 64, 34), (1, 65, 4, 2, 128, 35), (2, 77, 6, 2, 128, 36)]


def _bits(t):
    import torch
    return t.contiguous().view(torch.int16 if t.element_size() == 2 else torch.int32).cpu().numpy()


def _same(a, b, what):
    assert np.array_equal(_bits(a), _bits(b)), what


def _setup(B, T, Hq, Hkv, d, seed):
    import torch
    x = si.make_inputs(B, T, Hq, Hkv, d, seed, 1.0)
    dev = {n: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda() for n, a in x.items()}
    qkv = torch.empty((B, T, Hq + 2 * Hkv, d), dtype=torch.bfloat16, device="cuda")
    qkv[:, :, :Hq] = dev["q"]
    qkv[:, :, Hq:Hq + Hkv] = dev["k"]
    qkv[:, :, Hq + Hkv:] = dev["v"]
    torch.cuda.synchronize()
    views = (qkv[:, :, :Hq], qkv[:, :, Hq:Hq + Hkv], qkv[:, :, Hq + Hkv:])
    return dev, views


@pytest.mark.parametrize("B,T,Hq,Hkv,d,seed", SHAPES)
def test_packed_qkv_matches_contiguous(B, T, Hq, Hkv, d, seed):
    import torch
    print(f"strided B={B} T={T} Hq={Hq} Hkv={Hkv} d={d} seed={seed}", flush=True)
    scale = workload_scale(d)
    dev, (qv, kv, vv) = _setup(B, T, Hq, Hkv, d, seed)
    q, k, v, do = dev["q"], dev["k"], dev["v"], dev["do"]
    assert not qv.is_contiguous() and qv.stride()[1] == (Hq + 2 * Hkv) * d

    # forward: contiguous reference, then packed inputs with o in a padded buffer
    o_ref, lse_ref = cg.attn_fwd(q, k, v, scale=scale)
    pad = 64
    obuf = torch.full((B, T, Hq * d + pad), float("nan"), dtype=torch.bfloat16, device="cuda")
    o_view = obuf[:, :, :Hq * d].view(B, T, Hq, d)
    o_s, lse_s = cg.attn_fwd(qv, kv, vv, scale=scale, o=o_view)
    torch.cuda.synchronize()
    _same(o_s, o_ref, "o")
    _same(lse_s, lse_ref, "lse")
    assert torch.isnan(obuf[:, :, Hq * d:].float()).all(), "o padding overwritten"

    # backward with fp32 gradients: contiguous reference, then packed inputs and a packed
    # fp32 dQKV output buffer that starts out NaN everywhere
    delta_ref, dq_ref = cg.attn_bwd_dq(q, k, v, o_ref, do, lse_ref, scale=scale)
    dk_ref, dv_ref = cg.attn_bwd_dkv(q, k, v, do, lse_ref, delta_ref, scale=scale)
    dqkv = torch.full((B, T, Hq + 2 * Hkv, d), float("nan"), dtype=torch.float32, device="cuda")
    dqv, dkv_, dvv = dqkv[:, :, :Hq], dqkv[:, :, Hq:Hq + Hkv], dqkv[:, :, Hq + Hkv:]
    delta_s, _ = cg.attn_bwd_dq(qv, kv, vv, o_view, do, lse_s, scale=scale, dq=dqv)
    torch.cuda.synchronize()
    _same(delta_s, delta_ref, "delta")
    _same(dqv, dq_ref, "dq (packed fp32)")
    assert torch.isnan(dqkv[:, :, Hq:]).all(), "dq wrote outside its columns"
    cg.attn_bwd_dkv(qv, kv, vv, do, lse_s, delta_s, scale=scale, dk=dkv_, dv=dvv)
    torch.cuda.synchronize()
    _same(dkv_, dk_ref, "dk (packed fp32)")
    _same(dvv, dv_ref, "dv (packed fp32)")
    _same(dqv, dq_ref, "dq kept")

    # bf16 gradients into a packed bf16 buffer: the fp32 values rounded to nearest even
    g16 = torch.full((B, T, Hq + 2 * Hkv, d), float("nan"), dtype=torch.bfloat16, device="cuda")
    _, dq16 = cg.attn_bwd_dq(qv, kv, vv, o_view, do, lse_s, scale=scale, dq=g16[:, :, :Hq])
    dk16, dv16 = cg.attn_bwd_dkv(qv, kv, vv, do, lse_s, delta_s, scale=scale,
                                 dk=g16[:, :, Hq:Hq + Hkv], dv=g16[:, :, Hq + Hkv:])
    torch.cuda.synchronize()
    _same(dq16, dq_ref.to(torch.bfloat16), "dq bf16")
    _same(dk16, dk_ref.to(torch.bfloat16), "dk bf16")
    _same(dv16, dv_ref.to(torch.bfloat16), "dv bf16")

    # contiguous bf16 gradients (the strided call with contiguous strides)
    _, dq16c = cg.attn_bwd_dq(q, k, v, o_ref, do, lse_ref, scale=scale, grad_dtype=torch.bfloat16)
    dk16c, dv16c = cg.attn_bwd_dkv(q, k, v, do, lse_ref, delta_ref, scale=scale, grad_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    _same(dq16c, dq16, "dq bf16 contiguous")
    _same(dk16c, dk16, "dk bf16 contiguous")
    _same(dv16c, dv16, "dv bf16 contiguous")


# Tolerance of bf16 gradients against the oracle: the fp32 value g is within MAX_ABS of the
# exact r (and within REL_L2 in relative L2); rounding g to bf16 moves it by at most u |g|,
# u = 2^-8 the unit roundoff of 8 significant bits, so |bf16(g) - r| <= MAX_ABS + u (|r| +
# MAX_ABS) element-wise and the relative L2 error grows by at most u (1 + REL_L2).
BF16_UNIT_ROUNDOFF = 2.0 ** -8


@pytest.mark.parametrize("B,T,Hq,Hkv,d,seed", SHAPES[::2])
def test_bf16_gradients_against_oracle(B, T, Hq, Hkv, d, seed):
    import torch
    print(f"bf16 grads vs oracle B={B} T={T} Hq={Hq} Hkv={Hkv} d={d} seed={seed}", flush=True)
    scale = workload_scale(d)
    x = si.make_inputs(B, T, Hq, Hkv, d, seed, 1.0)
    want = oracle_run(x, scale)
    dev, (qv, kv, vv) = _setup(B, T, Hq, Hkv, d, seed)
    o, lse = cg.attn_fwd(qv, kv, vv, scale=scale)
    g16 = torch.empty((B, T, Hq + 2 * Hkv, d), dtype=torch.bfloat16, device="cuda")
    delta, dq = cg.attn_bwd_dq(qv, kv, vv, o, dev["do"], lse, scale=scale, dq=g16[:, :, :Hq])
    dk, dv = cg.attn_bwd_dkv(qv, kv, vv, dev["do"], lse, delta, scale=scale,
                             dk=g16[:, :, Hq:Hq + Hkv], dv=g16[:, :, Hq + Hkv:])
    torch.cuda.synchronize()
    for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        got = t.float().cpu().numpy().astype(np.float64)
        r = want[name]
        err = np.abs(got - r)
        bound = MAX_ABS + BF16_UNIT_ROUNDOFF * (np.abs(r) + MAX_ABS)
        assert np.all(err <= bound), (name, tuple(np.argwhere(err > bound)[0]), float(err.max()))
        rel = np.linalg.norm(got - r) / np.linalg.norm(r)
        assert rel <= REL_L2 + BF16_UNIT_ROUNDOFF * (1 + REL_L2), (name, rel)
