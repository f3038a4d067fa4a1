"""The C-ABI library on a host without a GPU: it loads, exports every entry point that
include/cgqa.h declares, and rejects bad arguments with the documented codes before
making any HIP call (so these checks run here, on the CPU)."""
import os
import re

import pytest

import causal_gqa_flash_amd as cg

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "cgqa.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b((?:attn|cgqa)_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = cg.library()
    names = declared_functions()
    assert {"attn_fwd", "attn_bwd_dq", "attn_bwd_dkv", "attn_status_string"} <= set(names)
    for name in names:
        assert hasattr(lib, name), name


def test_status_strings():
    for code in (cg.CGQA_OK, cg.CGQA_EINVAL, cg.CGQA_EUNSUPPORTED, cg.CGQA_EHIP, 99):
        s = cg.attn_status_string(code)
        assert isinstance(s, str) and s
    assert cg.library().cgqa_last_hip_error() == 0


# Distinct, 16-byte aligned, non-overlapping fake addresses: never dereferenced, because
# every call below is rejected by validation before any HIP call.
BASE = 1 << 40
SPACING = 1 << 36


def fake(i):
    return BASE + i * SPACING


GOOD = dict(B=1, T=64, Hq=6, Hkv=2, d=64, scale=0.125)


def call_fwd(ptrs=None, **kw):
    a = dict(GOOD, **kw)
    p = ptrs or [fake(i) for i in range(5)]
    return cg.library().attn_fwd(*p, a["B"], a["T"], a["Hq"], a["Hkv"], a["d"], a["scale"], None)


# The backward calls take 9 pointers: dq: q k v o dO lse | delta dO_absmax dq;
# dkv: q k v dO lse delta dO_absmax | dk dv.
def call_dq(ptrs=None, **kw):
    a = dict(GOOD, **kw)
    p = ptrs or [fake(i) for i in range(9)]
    return cg.library().attn_bwd_dq(*p, a["B"], a["T"], a["Hq"], a["Hkv"], a["d"], a["scale"], None)


def call_dkv(ptrs=None, **kw):
    a = dict(GOOD, **kw)
    p = ptrs or [fake(i) for i in range(9)]
    return cg.library().attn_bwd_dkv(*p, a["B"], a["T"], a["Hq"], a["Hkv"], a["d"], a["scale"], None)


BAD_SHAPES = [
    (dict(B=-1), cg.CGQA_EINVAL),
    (dict(T=-5), cg.CGQA_EINVAL),
    (dict(Hq=0), cg.CGQA_EINVAL),
    (dict(Hkv=0), cg.CGQA_EINVAL),
    (dict(Hq=6, Hkv=4), cg.CGQA_EINVAL),
    (dict(scale=0.0), cg.CGQA_EINVAL),
    (dict(scale=-0.125), cg.CGQA_EINVAL),
    (dict(scale=float("inf")), cg.CGQA_EINVAL),
    (dict(scale=float("nan")), cg.CGQA_EINVAL),
    (dict(d=32), cg.CGQA_EUNSUPPORTED),
    (dict(d=96), cg.CGQA_EUNSUPPORTED),
    (dict(d=256), cg.CGQA_EUNSUPPORTED),
    (dict(B=1 << 14, T=1 << 12, Hq=8, Hkv=8, d=64), cg.CGQA_EINVAL),   # 2^31 elements
]


@pytest.mark.parametrize("call", [call_fwd, call_dq, call_dkv])
@pytest.mark.parametrize("kw,code", BAD_SHAPES)
def test_bad_shapes_rejected(call, kw, code):
    assert call(**kw) == code


@pytest.mark.parametrize("call,n", [(call_fwd, 5), (call_dq, 9), (call_dkv, 9)])
def test_null_pointers_rejected(call, n):
    for i in range(n):
        p = [fake(j) for j in range(n)]
        p[i] = None
        assert call(ptrs=p) == cg.CGQA_EINVAL, i


@pytest.mark.parametrize("call,n", [(call_fwd, 5), (call_dq, 9), (call_dkv, 9)])
def test_misaligned_pointers_rejected(call, n):
    for i in range(n):
        p = [fake(j) for j in range(n)]
        p[i] += 8
        assert call(ptrs=p) == cg.CGQA_EUNSUPPORTED, i


@pytest.mark.parametrize("call,n,outs", [(call_fwd, 5, (3, 4)), (call_dq, 9, (6, 7, 8)),
                                         (call_dkv, 9, (7, 8))])
def test_overlapping_outputs_rejected(call, n, outs):
    for o in outs:
        for other in range(n):
            if other == o:
                continue
            p = [fake(j) for j in range(n)]
            p[o] = p[other] + 16          # inside the other buffer (the smallest, dO_absmax, is 48 bytes)
            assert call(ptrs=p) == cg.CGQA_EINVAL, (o, other)


@pytest.mark.parametrize("call", [call_fwd, call_dq, call_dkv])
def test_empty_problem_is_a_no_op(call):
    # Empty problems succeed without a HIP call, also with null pointers.
    assert call(B=0) == cg.CGQA_OK
    assert call(T=0) == cg.CGQA_OK
    assert call(ptrs=[None] * (5 if call is call_fwd else 9), T=0) == cg.CGQA_OK
    assert call(B=0, d=32) == cg.CGQA_EUNSUPPORTED   # shape errors still win


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    from causal_gqa_flash_amd import _binding
    monkeypatch.setattr(_binding, "_lib", None)
    monkeypatch.setattr(_binding, "HERE", str(tmp_path))
    with pytest.raises(ImportError):
        _binding.library()


# ---- strided entry points (every call below is rejected before any HIP call)

def strides(a, **kw):
    Hq, Hkv, d = a["Hq"], a["Hkv"], a["d"]
    s = dict(q_rs=Hq * d, kv_rs=Hkv * d, o_rs=Hq * d, do_rs=Hq * d, dq_rs=Hq * d, dkv_rs=Hkv * d, grad=0)
    s.update(kw)
    return s


def call_fwd_s(ptrs=None, st=None, **kw):
    a = dict(GOOD, **kw)
    s = strides(a, **(st or {}))
    p = ptrs or [fake(i) for i in range(5)]
    return cg.library().attn_fwd_strided(*p, a["B"], a["T"], a["Hq"], a["Hkv"], a["d"],
                                         s["q_rs"], s["kv_rs"], s["o_rs"], a["scale"], None)


def call_dq_s(ptrs=None, st=None, **kw):
    a = dict(GOOD, **kw)
    s = strides(a, **(st or {}))
    p = ptrs or [fake(i) for i in range(9)]
    return cg.library().attn_bwd_dq_strided(*p, a["B"], a["T"], a["Hq"], a["Hkv"], a["d"], s["q_rs"],
                                            s["kv_rs"], s["o_rs"], s["do_rs"], s["dq_rs"], s["grad"],
                                            a["scale"], None)


def call_dkv_s(ptrs=None, st=None, **kw):
    a = dict(GOOD, **kw)
    s = strides(a, **(st or {}))
    p = ptrs or [fake(i) for i in range(9)]
    return cg.library().attn_bwd_dkv_strided(*p, a["B"], a["T"], a["Hq"], a["Hkv"], a["d"], s["q_rs"],
                                             s["kv_rs"], s["do_rs"], s["dkv_rs"], s["grad"], a["scale"], None)


STRIDED = [(call_fwd_s, 5, (3, 4)), (call_dq_s, 9, (6, 7, 8)), (call_dkv_s, 9, (7, 8))]


@pytest.mark.parametrize("call", [c for c, _, _ in STRIDED])
@pytest.mark.parametrize("kw,code", BAD_SHAPES)
def test_strided_bad_shapes_rejected(call, kw, code):
    assert call(**kw) == code


@pytest.mark.parametrize("call,n,outs", STRIDED)
def test_strided_null_misaligned_overlapping_rejected(call, n, outs):
    for i in range(n):
        p = [fake(j) for j in range(n)]
        p[i] = None
        assert call(ptrs=p) == cg.CGQA_EINVAL, i
        p = [fake(j) for j in range(n)]
        p[i] += 8
        assert call(ptrs=p) == cg.CGQA_EUNSUPPORTED, i
    for o in outs:
        for other in range(n):
            if other != o:
                p = [fake(j) for j in range(n)]
                p[o] = p[other] + 16
                assert call(ptrs=p) == cg.CGQA_EINVAL, (o, other)


# (call, stride name, row width in elements (Hq*d = 384, Hkv*d = 128), alignment)
STRIDE_ARGS = [(call_fwd_s, "q_rs", 384, 8), (call_fwd_s, "kv_rs", 128, 8), (call_fwd_s, "o_rs", 384, 4),
               (call_dq_s, "q_rs", 384, 8), (call_dq_s, "kv_rs", 128, 8), (call_dq_s, "o_rs", 384, 8),
               (call_dq_s, "do_rs", 384, 8), (call_dq_s, "dq_rs", 384, 4),
               (call_dkv_s, "q_rs", 384, 8), (call_dkv_s, "kv_rs", 128, 8), (call_dkv_s, "do_rs", 384, 8),
               (call_dkv_s, "dkv_rs", 128, 4)]


@pytest.mark.parametrize("call,name,width,align", STRIDE_ARGS)
def test_bad_strides_rejected(call, name, width, align):
    assert call(st={name: width - 8}) == cg.CGQA_EINVAL           # shorter than its row
    assert call(st={name: -width}) == cg.CGQA_EINVAL
    assert call(st={name: width + align // 2}) == cg.CGQA_EUNSUPPORTED   # not whole units
    # B*T*rs reaches 2^31 elements
    assert call(st={name: 1 << 15}, B=1, T=1 << 16) == cg.CGQA_EINVAL
    # the empty problem still checks its strides
    assert call(st={name: width - 8}, T=0) == cg.CGQA_EINVAL


@pytest.mark.parametrize("call", [call_dq_s, call_dkv_s])
def test_unknown_gradient_type_rejected(call):
    for g in (-1, 2, 7):
        assert call(st={"grad": g}) == cg.CGQA_EINVAL


def test_packed_gradients_must_not_share_columns():
    # dk and dv in one buffer with row stride R = (Hq + 2 Hkv) d = 640 floats: dv placed
    # 64 bytes after dk lies inside dk's 128 columns of every row.
    R = 640
    p = [fake(j) for j in range(9)]
    p[8] = p[7] + 64
    assert call_dkv_s(ptrs=p, st={"dkv_rs": R}) == cg.CGQA_EINVAL
    # bf16 dv one row-window too far: its columns [96, 224) meet dk's [0, 128)
    p[8] = p[7] + 2 * 96
    assert call_dkv_s(ptrs=p, st={"dkv_rs": R, "grad": 1}) == cg.CGQA_EINVAL
    # dq written into the input q buffer's rows (q's columns) is an overlap
    p = [fake(j) for j in range(9)]
    p[8] = p[0] + 16
    assert call_dq_s(ptrs=p, st={"q_rs": 640, "dq_rs": 320}) == cg.CGQA_EINVAL


# ---- naive attention (the GPU reference mode). Every call below is rejected too.
def naive_need(a):
    return a["B"] * a["Hq"] * a["T"] * a["T"] * 4


def call_nfwd(ptrs=None, ws_bytes=None, **kw):
    a = dict(GOOD, **kw)
    p = ptrs or [fake(i) for i in range(6)]
    n = naive_need(a) if ws_bytes is None else ws_bytes
    return cg.library().attn_naive_fwd(*p[:5], p[5], n, a["B"], a["T"], a["Hq"], a["Hkv"], a["d"],
                                       a["scale"], None)


def call_nbwd(ptrs=None, ws_bytes=None, **kw):
    a = dict(GOOD, **kw)
    p = ptrs or [fake(i) for i in range(9)]
    n = naive_need(a) if ws_bytes is None else ws_bytes
    return cg.library().attn_naive_bwd(*p[:8], p[8], n, a["B"], a["T"], a["Hq"], a["Hkv"], a["d"],
                                       a["scale"], None)


NAIVE_BAD_SHAPES = [s for s in BAD_SHAPES if "d" not in s[0]] + [
    (dict(d=0), cg.CGQA_EUNSUPPORTED),
    (dict(d=129), cg.CGQA_EUNSUPPORTED),
    (dict(d=256), cg.CGQA_EUNSUPPORTED),
]


def test_naive_workspace_bytes():
    assert cg.attn_naive_workspace_bytes(16, 1024, 6) == 16 * 6 * 1024 * 1024 * 4
    assert cg.attn_naive_workspace_bytes(0, 64, 6) == 0
    assert cg.attn_naive_workspace_bytes(-1, 64, 6) == 0
    assert cg.attn_naive_workspace_bytes(1, 64, 0) == 0
    assert cg.attn_naive_workspace_bytes(1 << 16, 1 << 12, 8) == 0   # 2^31 rows
    assert cg.attn_naive_workspace_bytes(1 << 14, 1 << 12, 8) == (1 << 29) * (1 << 12) * 4


@pytest.mark.parametrize("call", [call_nfwd, call_nbwd])
@pytest.mark.parametrize("kw,code", NAIVE_BAD_SHAPES)
def test_naive_bad_shapes_rejected(call, kw, code):
    a = dict(GOOD, **kw)
    ws = max(0, naive_need(a)) if a["B"] >= 0 and a["T"] >= 0 and a["Hq"] >= 1 else 0
    assert call(ws_bytes=ws, **kw) == code


@pytest.mark.parametrize("call", [call_nfwd, call_nbwd])
def test_naive_small_or_missing_workspace_rejected(call):
    need = naive_need(GOOD)
    assert call(ws_bytes=need - 1) == cg.CGQA_EINVAL
    assert call(ws_bytes=0) == cg.CGQA_EINVAL
    n = 6 if call is call_nfwd else 9
    p = [fake(j) for j in range(n)]
    p[-1] = None
    assert call(ptrs=p) == cg.CGQA_EINVAL


@pytest.mark.parametrize("call,n", [(call_nfwd, 6), (call_nbwd, 9)])
def test_naive_null_and_misaligned_rejected(call, n):
    for i in range(n):
        p = [fake(j) for j in range(n)]
        p[i] = None
        assert call(ptrs=p) == cg.CGQA_EINVAL, i
        p = [fake(j) for j in range(n)]
        p[i] += 4
        assert call(ptrs=p) == cg.CGQA_EUNSUPPORTED, i


@pytest.mark.parametrize("call,n,outs", [(call_nfwd, 6, (3, 4, 5)), (call_nbwd, 9, (4, 5, 6, 7, 8))])
def test_naive_overlaps_rejected(call, n, outs):
    for o in outs:
        for other in range(n):
            if other == o:
                continue
            p = [fake(j) for j in range(n)]
            p[o] = p[other] + 64
            assert call(ptrs=p) == cg.CGQA_EINVAL, (o, other)


@pytest.mark.parametrize("call", [call_nfwd, call_nbwd])
def test_naive_empty_problem_is_a_no_op(call):
    n = 6 if call is call_nfwd else 9
    assert call(ptrs=[None] * n, ws_bytes=0, T=0) == cg.CGQA_OK
    assert call(ptrs=[None] * n, ws_bytes=0, B=0) == cg.CGQA_OK


# ---- the projection matmul. Every call below is rejected too.
def call_gemm(ptrs=None, M=64, N=64, K=64, flags=0, ws=None, ws_bytes=0):
    p = ptrs or [fake(i) for i in range(4)]
    return cg.library().cgqa_gemm(p[0], p[1], p[2], p[3], M, N, K, flags, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,code", [
    (dict(M=-1), cg.CGQA_EINVAL), (dict(N=-1), cg.CGQA_EINVAL), (dict(K=-32), cg.CGQA_EINVAL),
    (dict(flags=8), cg.CGQA_EINVAL), (dict(flags=-1), cg.CGQA_EINVAL),
    (dict(K=48), cg.CGQA_EUNSUPPORTED), (dict(K=1), cg.CGQA_EUNSUPPORTED),
    (dict(M=12, flags=cg.CGQA_GEMM_A_KM), cg.CGQA_EUNSUPPORTED),
    (dict(N=20, flags=cg.CGQA_GEMM_B_KN), cg.CGQA_EUNSUPPORTED),
    (dict(M=1 << 16, K=1 << 15), cg.CGQA_EINVAL), (dict(N=1 << 16, K=1 << 15), cg.CGQA_EINVAL),
    (dict(M=1 << 16, N=1 << 15), cg.CGQA_EINVAL),
])
def test_gemm_bad_sizes_rejected(kw, code):
    assert call_gemm(**kw) == code


def test_gemm_bad_pointers_rejected():
    for i in range(3):                         # A, B, C; R may be null
        p = [fake(j) for j in range(4)]
        p[i] = None
        assert call_gemm(ptrs=p) == cg.CGQA_EINVAL, i
    for i in range(4):
        p = [fake(j) for j in range(4)]
        p[i] += 8
        assert call_gemm(ptrs=p) == cg.CGQA_EUNSUPPORTED, i
    # C overlapping A or B, or R overlapping C without being C
    for other in (0, 1, 3):
        p = [fake(j) for j in range(4)]
        p[2] = p[other] + 64
        assert call_gemm(ptrs=p) == cg.CGQA_EINVAL, other
    # R == C needs an fp32 C
    p = [fake(j) for j in range(4)]
    p[3] = p[2]
    assert call_gemm(ptrs=p, flags=cg.CGQA_GEMM_C_BF16) == cg.CGQA_EINVAL


def test_gemm_empty_is_a_no_op():
    assert call_gemm(ptrs=[None] * 4, M=0) == cg.CGQA_OK
    assert call_gemm(ptrs=[None] * 4, N=0) == cg.CGQA_OK


def test_gemm_workspace_rules():
    # misaligned or overlapping workspaces are rejected before any HIP call
    assert call_gemm(ws=fake(5) + 8, ws_bytes=1 << 20) == cg.CGQA_EUNSUPPORTED
    for other in range(4):
        assert call_gemm(ws=fake(other) + 64, ws_bytes=1 << 20) == cg.CGQA_EINVAL, other
    # size query: long K over few tiles splits; many tiles or short K do not
    assert cg.gemm_workspace_bytes(640, 384, 16384) == 32 * 640 * 384 * 4
    assert cg.gemm_workspace_bytes(1, 1, 1024) == 4 * 4 * 4          # slices padded to 4 floats
    assert cg.gemm_workspace_bytes(16384, 640, 384) == 0
    assert cg.gemm_workspace_bytes(640, 384, 256) == 0
    assert cg.gemm_workspace_bytes(640, 384, 100) == 0



# ---- rotary embedding. Every call below is rejected too.
def call_rope(ptrs=None, B=1, T=64, Hq=6, Hkv=2, d=64, rs=None):
    p = ptrs or [fake(i) for i in range(6)]
    r = rs or [Hq * d, Hkv * d, Hq * d, Hkv * d]
    return cg.library().attn_rope_qk(*p, B, T, Hq, Hkv, d, *r, None)


def test_rope_rejections():
    for i in range(6):
        p = [fake(j) for j in range(6)]
        p[i] = None
        assert call_rope(ptrs=p) == cg.CGQA_EINVAL, i
        p = [fake(j) for j in range(6)]
        p[i] += 8
        assert call_rope(ptrs=p) == cg.CGQA_EUNSUPPORTED, i
    assert call_rope(d=96) == cg.CGQA_EUNSUPPORTED
    assert call_rope(Hq=6, Hkv=4) == cg.CGQA_EINVAL
    assert call_rope(rs=[6 * 64 - 8, 128, 384, 128]) == cg.CGQA_EINVAL         # stride shorter than a row
    assert call_rope(rs=[6 * 64 + 4, 128, 384, 128]) == cg.CGQA_EUNSUPPORTED   # not a multiple of 8
    # outputs overlapping something other than their own input, at the same place
    for o in (2, 3):
        for other in range(6):
            if other == o:
                continue
            p = [fake(j) for j in range(6)]
            p[o] = p[other] + 64
            assert call_rope(ptrs=p) == cg.CGQA_EINVAL, (o, other)
    # in place with a different stride is an overlap
    p = [fake(j) for j in range(6)]
    p[2] = p[0]
    assert call_rope(ptrs=p, rs=[384, 128, 392, 128]) == cg.CGQA_EINVAL
    assert call_rope(ptrs=[None] * 6, T=0) == cg.CGQA_OK


def test_rope_backward_rejections():
    lib = cg.library()
    args = (1, 64, 6, 2, 64, 0.125, None)
    p = [fake(j) for j in range(11)]
    for fn in (lib.attn_bwd_dq_rope, lib.attn_bwd_dkv_rope):
        for i in (9, 10):                      # missing table
            q = list(p)
            q[i] = None
            assert fn(*q, *args) == cg.CGQA_EINVAL, i
        q = list(p)
        q[9] += 8                               # misaligned table
        assert fn(*q, *args) == cg.CGQA_EUNSUPPORTED
        q = list(p)
        q[9] = q[8] + 64                        # table inside an output
        assert fn(*q, *args) == cg.CGQA_EINVAL


def test_rope_forward_rejections():
    """attn_fwd_rope: q k v o lse cos sin; the forward's own checks, then the tables'."""
    lib = cg.library()
    p = [fake(j) for j in range(7)]

    def call(ptrs, B=1, T=64, Hq=6, Hkv=2, d=64):
        return lib.attn_fwd_rope(*ptrs, B, T, Hq, Hkv, d, 0.125, None)

    for i in range(7):
        q = list(p)
        q[i] = None
        assert call(q) == cg.CGQA_EINVAL, i
        q = list(p)
        q[i] += 8
        assert call(q) == cg.CGQA_EUNSUPPORTED, i
    assert call(p, d=128) == cg.CGQA_EUNSUPPORTED          # d = 64 only
    assert call(p, Hq=6, Hkv=4) == cg.CGQA_EINVAL
    for t in (5, 6):                                        # a table inside an output
        for out in (3, 4):
            q = list(p)
            q[t] = q[out] + 64
            assert call(q) == cg.CGQA_EINVAL, (t, out)
    assert call([None] * 7, T=0) == cg.CGQA_OK


def test_gemm_static_rejects_shapes_beyond_its_scratch():
    """cgqa_gemm_static keeps split-K partials in a fixed device array: a shape whose
    split needs more is CGQA_EINVAL before any HIP call; the usual rules still apply."""
    lib = cg.library()
    p = [fake(j) for j in range(4)]
    assert lib.cgqa_gemm_workspace_bytes(1024, 1024, 8192) > (16 << 20)
    assert lib.cgqa_gemm_static(*p, 1024, 1024, 8192, 0, None) == cg.CGQA_EINVAL
    assert lib.cgqa_gemm_static(*p, 256, 384, 100, 0, None) == cg.CGQA_EUNSUPPORTED   # K % 32
    assert lib.cgqa_gemm_static(p[0], p[1], None, None, 256, 384, 8192, 0, None) == cg.CGQA_EINVAL
    assert lib.cgqa_gemm_static(*p, 0, 384, 8192, 0, None) == cg.CGQA_OK             # empty


def test_calib_rejections():
    lib = cg.library()
    s, c = fake(0), fake(1)
    for blocks, iters in ((0, 10), (1 << 17, 10), (4, 0), (4, (1 << 20) + 1)):
        assert lib.cgqa_calib_mfma(s, c, blocks, iters, None, None) == cg.CGQA_EINVAL
    assert lib.cgqa_calib_mfma(None, c, 4, 10, None, None) == cg.CGQA_EINVAL
    assert lib.cgqa_calib_mfma(s + 8, c, 4, 10, None, None) == cg.CGQA_EUNSUPPORTED
    assert lib.cgqa_calib_mfma(s, c + 8, 4, 10, None, None) == cg.CGQA_EUNSUPPORTED
    assert lib.cgqa_calib_mfma(s, s + 64, 4, 10, None, None) == cg.CGQA_EINVAL   # clocks inside sink
