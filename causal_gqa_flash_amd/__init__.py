"""causal_gqa_flash_amd: causal grouped-query flash attention on AMD MI355X (gfx950).

Thin Python binding over the C-ABI library ``libcgqa.so`` (declared in
``include/cgqa.h``). Every step of the computation runs in the library's HIP
kernels; this module only checks tensor metadata, allocates outputs with torch and
passes raw device pointers and the current HIP stream. If the library is missing
the calls raise: there is no fallback.
"""
from ._binding import (  # noqa: F401
    CGQA_EHIP,
    CGQA_EINVAL,
    CGQA_EUNSUPPORTED,
    CGQA_GEMM_A_KM,
    CGQA_GEMM_B_KN,
    CGQA_GEMM_C_BF16,
    CGQA_GRAD_BF16,
    CGQA_GRAD_F32,
    CGQA_OK,
    CgqaError,
    attn_bwd_dkv,
    attn_bwd_dq,
    attn_fwd,
    attn_naive_bwd,
    attn_naive_fwd,
    attn_naive_workspace_bytes,
    attn_status_string,
    bwd_delta,
    calib_mfma,
    gemm,
    gemm_workspace_bytes,
    library,
    library_path,
    rope_qk,
)
