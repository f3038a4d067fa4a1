"""The projection matmul (cgqa_gemm) through the C-ABI against the fp64 oracle.

Bound: C is a sum of K products (exact in fp32) plus R, added in fp32 in some order, so
|c - c_exact| <= (K + 2) u S with u = 2^-24 and S = sum_k |a||b| + |r| (the classic bound
for any summation order). A bf16 C adds its own rounding, at most 2^-8 of the value."""
import itertools

import numpy as np
import pytest

import causal_gqa_flash_amd as cg
import synthetic_inputs as si
from oracle import gemm as og

pytestmark = pytest.mark.gpu

U32, U16 = 2.0 ** -24, 2.0 ** -8


def _bits(rng, shape, scale=1.0):
    return si.f32_to_bf16_bits(rng.standard_normal(shape, dtype=np.float32) * np.float32(scale))


def _dev(bits):
    import torch
    return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).cuda()


def _check(got, want, S, K, bf16, what):
    b32 = (K + 2) * U32 * S
    bound = b32 * (1 + U16) + U16 * np.abs(want) if bf16 else b32
    bound = bound + 1e-30
    err = np.abs(got - want)
    assert np.all(err <= bound), (what, tuple(np.argwhere(err > bound)[0]), float((err / bound).max()))


def _run(a, b, r, M, N, K, a_km, b_kn, c_bf16, r_mode, ws_bytes=0):
    import torch
    da, db = _dev(a), _dev(b)
    out_dtype = torch.bfloat16 if c_bf16 else torch.float32
    ws = torch.empty((ws_bytes // 4,), dtype=torch.float32, device="cuda") if ws_bytes else None
    if r_mode == "none":
        c = cg.gemm(da, db, a_km=a_km, b_kn=b_kn, out_dtype=out_dtype, workspace=ws)
    elif r_mode == "separate":
        c = cg.gemm(da, db, r=torch.from_numpy(r).cuda(), a_km=a_km, b_kn=b_kn, out_dtype=out_dtype,
                    workspace=ws)
    else:   # C += A B^T: R is C itself
        c = torch.from_numpy(r).cuda()
        cg.gemm(da, db, r=c, c=c, a_km=a_km, b_kn=b_kn, workspace=ws)
    torch.cuda.synchronize()
    return c.float().cpu().numpy().astype(np.float64)


SHAPES = [(1, 1, 32), (33, 40, 96), (136, 200, 64), (130, 264, 96), (256, 136, 32), (8, 8, 0)]
CASES = [(s, akm, bkn, cbf, rm) for s in SHAPES for akm, bkn in itertools.product((False, True), repeat=2)
         for cbf in (False, True) for rm in ("none", "separate", "inplace")
         if not (akm and s[0] % 8) and not (bkn and s[1] % 8) and not (cbf and rm == "inplace")]


@pytest.mark.parametrize("shape,a_km,b_kn,c_bf16,r_mode", CASES)
def test_gemm_matches_oracle(shape, a_km, b_kn, c_bf16, r_mode):
    M, N, K = shape
    print(f"gemm M={M} N={N} K={K} a_km={a_km} b_kn={b_kn} bf16={c_bf16} r={r_mode}", flush=True)
    rng = np.random.default_rng(M * 131 + N * 7 + K)
    a = _bits(rng, (K, M) if a_km else (M, K))
    b = _bits(rng, (K, N) if b_kn else (N, K))
    r = rng.standard_normal((M, N)).astype(np.float32)
    got = _run(a, b, r, M, N, K, a_km, b_kn, c_bf16, r_mode)
    rr = None if r_mode == "none" else r.astype(np.float64)
    want = og.gemm(a, b, rr, a_km=a_km, b_kn=b_kn)
    S = og.abs_product(a, b, a_km, b_kn) + (0.0 if rr is None else np.abs(rr))
    _check(got, want, S, K, c_bf16, "c")


# K split over several workgroups per tile (few tiles, long K), with the full workspace
# and with one that holds only three partial products.
SPLIT_SHAPES = [(136, 200, 2048), (8, 8, 512), (1, 1, 1024), (200, 136, 4096)]
SPLIT_CASES = [(s, akm, bkn, cbf, rm, full) for s in SPLIT_SHAPES
               for akm, bkn in itertools.product((False, True), repeat=2)
               for cbf in (False, True) for rm in ("none", "separate", "inplace") for full in (True, False)
               if not (akm and s[0] % 8) and not (bkn and s[1] % 8) and not (cbf and rm == "inplace")]


@pytest.mark.parametrize("shape,a_km,b_kn,c_bf16,r_mode,full", SPLIT_CASES)
def test_gemm_split_k_matches_oracle(shape, a_km, b_kn, c_bf16, r_mode, full):
    M, N, K = shape
    wsb = cg.gemm_workspace_bytes(M, N, K) if full else 3 * M * N * 4
    assert cg.gemm_workspace_bytes(M, N, K) > 0
    print(f"gemm split M={M} N={N} K={K} a_km={a_km} b_kn={b_kn} bf16={c_bf16} r={r_mode} ws={wsb}", flush=True)
    rng = np.random.default_rng(M * 31 + N * 3 + K + full)
    a = _bits(rng, (K, M) if a_km else (M, K))
    b = _bits(rng, (K, N) if b_kn else (N, K))
    r = rng.standard_normal((M, N)).astype(np.float32)
    got = _run(a, b, r, M, N, K, a_km, b_kn, c_bf16, r_mode, wsb)
    rr = None if r_mode == "none" else r.astype(np.float64)
    want = og.gemm(a, b, rr, a_km=a_km, b_kn=b_kn)
    S = og.abs_product(a, b, a_km, b_kn) + (0.0 if rr is None else np.abs(rr))
    _check(got, want, S, K, c_bf16, "c")


def test_split_k_repeatable():
    import torch
    rng = np.random.default_rng(14)
    M, N, K = 640, 384, 16384
    a, b = _dev(_bits(rng, (K, M))), _dev(_bits(rng, (K, N)))
    ws = torch.empty((cg.gemm_workspace_bytes(M, N, K) // 4,), dtype=torch.float32, device="cuda")
    c1 = cg.gemm(a, b, a_km=True, b_kn=True, workspace=ws)
    c2 = cg.gemm(a, b, a_km=True, b_kn=True, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(c1.view(torch.int32), c2.view(torch.int32))


def test_layouts_give_the_same_bits():
    import torch
    rng = np.random.default_rng(11)
    M, N, K = 264, 136, 96
    a = _bits(rng, (M, K))
    b = _bits(rng, (N, K))
    outs = []
    for a_km, b_kn in itertools.product((False, True), repeat=2):
        aa = np.ascontiguousarray(a.T) if a_km else a
        bb = np.ascontiguousarray(b.T) if b_kn else b
        c = cg.gemm(_dev(aa), _dev(bb), a_km=a_km, b_kn=b_kn)
        torch.cuda.synchronize()
        outs.append(c.cpu().numpy())
    for o in outs[1:]:
        assert np.array_equal(o.view(np.int32), outs[0].view(np.int32))


def test_gemm_repeatable():
    import torch
    rng = np.random.default_rng(12)
    a, b = _dev(_bits(rng, (1000, 384))), _dev(_bits(rng, (640, 384)))
    c1 = cg.gemm(a, b)
    c2 = cg.gemm(a, b)
    torch.cuda.synchronize()
    assert torch.equal(c1.view(torch.int32), c2.view(torch.int32))


def test_empty_sizes():
    import torch
    rng = np.random.default_rng(13)
    # K = 0 with R: C = R exactly; M or N = 0: nothing to do.
    r = torch.from_numpy(rng.standard_normal((40, 24)).astype(np.float32)).cuda()
    a = torch.empty((40, 0), dtype=torch.bfloat16, device="cuda")
    b = torch.empty((24, 0), dtype=torch.bfloat16, device="cuda")
    c = cg.gemm(a, b, r=r)
    torch.cuda.synchronize()
    assert torch.equal(c, r)
    z = cg.gemm(torch.empty((0, 32), dtype=torch.bfloat16, device="cuda"), _dev(_bits(rng, (8, 32))))
    assert z.shape == (0, 8)


# The projections of the attention half of a layer at B*T = 16384 tokens of the bench
# workload (model width 6*64 = 384; fused QKV width (6 + 2 + 2) * 64 = 640), forward and
# the backward's dX and dW (with its K split), checked on sampled rows of C (rows are
# independent).
MODEL = [("qkv", 16384, 640, 384, False, False, True, False),
         ("wo_residual", 16384, 384, 384, False, False, False, True),
         ("dx_qkv", 16384, 384, 640, False, True, False, False),
         ("dw_qkv", 640, 384, 16384, True, True, False, False)]


@pytest.mark.parametrize("name,M,N,K,a_km,b_kn,c_bf16,with_r", MODEL)
def test_gemm_projection_shapes_sampled(name, M, N, K, a_km, b_kn, c_bf16, with_r):
    import torch
    print(f"gemm projection {name} M={M} N={N} K={K}", flush=True)
    rng = np.random.default_rng(len(name) * 1000 + K)
    a = _bits(rng, (K, M) if a_km else (M, K))
    b = _bits(rng, (K, N) if b_kn else (N, K), 1.0 / np.sqrt(K))
    r = rng.standard_normal((M, N)).astype(np.float32) if with_r else None
    got = _run(a, b, r, M, N, K, a_km, b_kn, c_bf16, "separate" if with_r else "none",
               cg.gemm_workspace_bytes(M, N, K))
    rows = np.unique(np.concatenate([[0, M - 1], rng.integers(0, M, 62)]))
    a_rows = np.ascontiguousarray(a[:, rows]) if a_km else a[rows]
    rr = None if r is None else r[rows].astype(np.float64)
    want = og.gemm(a_rows, b, rr, a_km=a_km, b_kn=b_kn)
    S = og.abs_product(a_rows, b, a_km, b_kn) + (0.0 if rr is None else np.abs(rr))
    _check(got[rows], want, S, K, c_bf16, name)
