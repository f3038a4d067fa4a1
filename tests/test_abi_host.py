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


def call_dq(ptrs=None, **kw):
    a = dict(GOOD, **kw)
    p = ptrs or [fake(i) for i in range(8)]
    return cg.library().attn_bwd_dq(*p, a["B"], a["T"], a["Hq"], a["Hkv"], a["d"], a["scale"], None)


def call_dkv(ptrs=None, **kw):
    a = dict(GOOD, **kw)
    p = ptrs or [fake(i) for i in range(8)]
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


@pytest.mark.parametrize("call,n", [(call_fwd, 5), (call_dq, 8), (call_dkv, 8)])
def test_null_pointers_rejected(call, n):
    for i in range(n):
        p = [fake(j) for j in range(n)]
        p[i] = None
        assert call(ptrs=p) == cg.CGQA_EINVAL, i


@pytest.mark.parametrize("call,n", [(call_fwd, 5), (call_dq, 8), (call_dkv, 8)])
def test_misaligned_pointers_rejected(call, n):
    for i in range(n):
        p = [fake(j) for j in range(n)]
        p[i] += 8
        assert call(ptrs=p) == cg.CGQA_EUNSUPPORTED, i


@pytest.mark.parametrize("call,n,outs", [(call_fwd, 5, (3, 4)), (call_dq, 8, (6, 7)),
                                         (call_dkv, 8, (6, 7))])
def test_overlapping_outputs_rejected(call, n, outs):
    for o in outs:
        for other in range(n):
            if other == o:
                continue
            p = [fake(j) for j in range(n)]
            p[o] = p[other] + 64          # inside the other buffer
            assert call(ptrs=p) == cg.CGQA_EINVAL, (o, other)


@pytest.mark.parametrize("call", [call_fwd, call_dq, call_dkv])
def test_empty_problem_is_a_no_op(call):
    # Empty problems succeed without a HIP call, also with null pointers.
    assert call(B=0) == cg.CGQA_OK
    assert call(T=0) == cg.CGQA_OK
    assert call(ptrs=[None] * (5 if call is call_fwd else 8), T=0) == cg.CGQA_OK
    assert call(B=0, d=32) == cg.CGQA_EUNSUPPORTED   # shape errors still win


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    from causal_gqa_flash_amd import _binding
    monkeypatch.setattr(_binding, "_lib", None)
    monkeypatch.setattr(_binding, "HERE", str(tmp_path))
    with pytest.raises(ImportError):
        _binding.library()
