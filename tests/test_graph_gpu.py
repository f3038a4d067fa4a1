"""The calls under HIP graph capture: a training step's attention (rotation pass, forward,
backward with the gradients turned back) and a projection matmul, captured once with
torch.cuda.graph and replayed several times with unrelated eager work and
synchronisations in between; every replay gives the bits of the eager calls. The kernels
record no memset nodes (nothing is cleared on the device), so replays start from the
same state."""
import numpy as np
import pytest

import causal_gqa_flash_amd as cg
import synthetic_inputs as si
from parity_util import to_device

pytestmark = pytest.mark.gpu


def test_attention_step_replays_bit_exactly():
    import torch
    B, T, Hq, Hkv, d = 2, 300, 6, 2, 64
    x = si.make_inputs(B, T, Hq, Hkv, d, 61, 1.0)
    dev = to_device(x)
    c, s = si.rope_tables(T, d)
    rc, rs = torch.from_numpy(c).cuda(), torch.from_numpy(s).cuda()
    bf, f32 = dict(dtype=torch.bfloat16, device="cuda"), dict(dtype=torch.float32, device="cuda")
    qr, kr = torch.empty((B, T, Hq, d), **bf), torch.empty((B, T, Hkv, d), **bf)
    o, lse = torch.empty((B, T, Hq, d), **bf), torch.empty((B, Hq, T), **f32)
    delta, dq = cg.bwd_delta(B, Hq, T, device="cuda"), torch.empty((B, T, Hq, d), **f32)
    dk, dv = torch.empty((B, T, Hkv, d), **f32), torch.empty((B, T, Hkv, d), **f32)
    wq = torch.from_numpy(si.f32_to_bf16_bits(np.random.default_rng(62).standard_normal((640, 384), dtype=np.float32)).view(np.int16)).view(torch.bfloat16).cuda()
    xin = torch.from_numpy(si.f32_to_bf16_bits(np.random.default_rng(63).standard_normal((B * T, 384), dtype=np.float32)).view(np.int16)).view(torch.bfloat16).cuda()
    proj = torch.empty((B * T, 640), **f32)

    def step():
        cg.rope_qk(dev["q"], dev["k"], rc, rs, q_out=qr, k_out=kr)
        cg.attn_fwd(qr, kr, dev["v"], scale=0.125, o=o, lse=lse)
        cg.attn_bwd_dq(qr, kr, dev["v"], o, dev["do"], lse, scale=0.125, delta=delta, dq=dq, rope=(rc, rs))
        cg.attn_bwd_dkv(qr, kr, dev["v"], dev["do"], lse, delta, scale=0.125, dk=dk, dv=dv, rope=(rc, rs))
        cg.gemm(xin, wq, c=proj)

    outs = (qr, kr, o, lse, delta, dq, dk, dv, proj)
    step()
    torch.cuda.synchronize()
    eager = [t.clone() for t in outs]

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):       # warm-up on a side stream, as torch's capture wants
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for rep in range(4):
        for t in outs:
            t.fill_(float("nan") if t.dtype == torch.float32 else 0.0)
        junk = torch.randn(1 << 20, device="cuda").sum()   # unrelated eager work
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for got, want in zip(outs, eager):
            w = torch.int16 if got.element_size() == 2 else torch.int32
            assert torch.equal(got.view(w), want.view(w)), rep
        del junk
