"""The allocation-free GEMM entry point, cgqa_gemm_static, called through the C-ABI, against
cgqa_gemm given a workspace: bit for bit, on two calls in a row (the second on smaller
matrices, so the shared scratch still holds the first call's partials)."""
import ctypes

import pytest

import causal_gqa_flash_amd as cg

pytestmark = pytest.mark.gpu

# (M, N, K, flags): K splits 32 ways (12 MiB of partials), then 16 ways (2 MiB), the
# second with a bf16 C and B stored [K][N].
CALLS = [(256, 384, 8192, 0), (128, 256, 4096, cg.CGQA_GEMM_C_BF16 | cg.CGQA_GEMM_B_KN)]


def _inputs(M, N, K, flags, seed):
    import torch
    g = torch.Generator(device="cuda").manual_seed(seed)
    a = torch.randn(M, K, generator=g, device="cuda").bfloat16()
    b = torch.randn(*((K, N) if flags & cg.CGQA_GEMM_B_KN else (N, K)), generator=g, device="cuda").bfloat16()
    r = torch.randn(M, N, generator=g, device="cuda")
    cdt = torch.bfloat16 if flags & cg.CGQA_GEMM_C_BF16 else torch.float32
    return a, b, r, cdt


def test_static_scratch_matches_workspace_call():
    import torch
    lib = cg.library()
    stream = torch.cuda.current_stream().cuda_stream
    p = lambda t: ctypes.c_void_p(t.data_ptr())
    for i, (M, N, K, flags) in enumerate(CALLS):
        print(f"gemm_static call {i}: M={M} N={N} K={K} flags={flags}", flush=True)
        a, b, r, cdt = _inputs(M, N, K, flags, 90 + i)
        need = lib.cgqa_gemm_workspace_bytes(M, N, K)
        assert 0 < need <= cg.library().cgqa_gemm_workspace_bytes(256, 384, 8192)
        ws = torch.empty(need // 4, dtype=torch.float32, device="cuda")
        want = torch.empty(M, N, dtype=cdt, device="cuda")
        got = torch.full((M, N), float("nan"), dtype=cdt, device="cuda")
        assert lib.cgqa_gemm(p(a), p(b), p(want), p(r), M, N, K, flags, p(ws), need, ctypes.c_void_p(stream)) == 0
        assert lib.cgqa_gemm_static(p(a), p(b), p(got), p(r), M, N, K, flags, ctypes.c_void_p(stream)) == 0
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int16 if cdt == torch.bfloat16 else torch.int32),
                           want.view(torch.int16 if cdt == torch.bfloat16 else torch.int32)), (M, N, K)
        # and the product itself, against fp32 torch on the same bf16 inputs
        bm = b.float() if flags & cg.CGQA_GEMM_B_KN else b.float().t()
        ref = a.float() @ bm + r
        top = ref.abs().max().item()
        if cdt == torch.bfloat16:
            bound = ref.abs() * 2.0 ** -8 + 1e-4 * top      # one bf16 rounding of C
        else:
            bound = torch.full_like(ref, 1e-4 * top)        # fp32 sums in another order
        assert bool(((got.float() - ref).abs() <= bound).all()), (M, N, K)
