"""ctypes binding of libcgqa.so: argument marshalling only (see include/cgqa.h)."""
import ctypes
import math
import os

HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_NAME = "libcgqa.so"

CGQA_OK = 0
CGQA_EINVAL = 1
CGQA_EUNSUPPORTED = 2
CGQA_EHIP = 3
CGQA_GRAD_F32 = 0
CGQA_GRAD_BF16 = 1
CGQA_GEMM_A_KM = 1
CGQA_GEMM_B_KN = 2
CGQA_GEMM_C_BF16 = 4

_lib = None


class CgqaError(RuntimeError):
    def __init__(self, call, status, detail=""):
        self.status = status
        msg = f"{call} failed with status {status}: {attn_status_string(status)}"
        super().__init__(msg + (f" ({detail})" if detail else ""))


def library_path() -> str:
    return os.path.join(HERE, _LIB_NAME)


def library():
    """The loaded ctypes library. Raises if it has not been built: no fallback exists."""
    global _lib
    if _lib is None:
        path = library_path()
        if not os.path.exists(path):
            raise ImportError(f"{path} is missing: build it with "
                              "`python -c 'import __graft_entry__ as g; g.build()'`")
        lib = ctypes.CDLL(path)
        vp = ctypes.c_void_p
        i = ctypes.c_int
        f = ctypes.c_float
        lib.attn_fwd.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, vp]
        lib.attn_fwd.restype = i
        lib.attn_bwd_dq.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, vp]
        lib.attn_bwd_dq.restype = i
        lib.attn_bwd_dkv.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, vp]
        lib.attn_bwd_dkv.restype = i
        lib.attn_fwd_strided.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, i, i, f, vp]
        lib.attn_fwd_strided.restype = i
        lib.attn_bwd_dq_strided.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, i, i, i, i, f, vp]
        lib.attn_bwd_dq_strided.restype = i
        lib.attn_bwd_dkv_strided.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, i, i, i, f, vp]
        lib.attn_bwd_dkv_strided.restype = i
        sz = ctypes.c_size_t
        lib.attn_naive_workspace_bytes.argtypes = [i, i, i]
        lib.attn_naive_workspace_bytes.restype = sz
        lib.attn_naive_fwd.argtypes = [vp, vp, vp, vp, vp, vp, sz, i, i, i, i, i, f, vp]
        lib.attn_naive_fwd.restype = i
        lib.attn_naive_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, i, i, i, i, i, f, vp]
        lib.attn_naive_bwd.restype = i
        lib.cgqa_gemm.argtypes = [vp, vp, vp, vp, i, i, i, i, vp, ctypes.c_size_t, vp]
        lib.attn_rope_qk.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, i, i, vp]
        lib.attn_rope_qk.restype = i
        lib.attn_fwd_rope.argtypes = [vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, vp]
        lib.attn_fwd_rope.restype = i
        lib.attn_bwd_dq_rope.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, vp]
        lib.attn_bwd_dq_rope.restype = i
        lib.attn_bwd_dkv_rope.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, vp]
        lib.attn_bwd_dkv_rope.restype = i
        lib.cgqa_calib_mfma.argtypes = [vp, vp, i, i, ctypes.POINTER(ctypes.c_double), vp]
        lib.cgqa_calib_mfma.restype = i
        lib.cgqa_gemm_static.argtypes = [vp, vp, vp, vp, i, i, i, i, vp]
        lib.cgqa_gemm_static.restype = i
        lib.cgqa_gemm_workspace_bytes.argtypes = [i, i, i]
        lib.cgqa_gemm_workspace_bytes.restype = ctypes.c_size_t
        lib.cgqa_gemm.restype = i
        lib.attn_status_string.argtypes = [i]
        lib.attn_status_string.restype = ctypes.c_char_p
        lib.cgqa_last_hip_error.argtypes = []
        lib.cgqa_last_hip_error.restype = i
        _lib = lib
    return _lib


def attn_status_string(status: int) -> str:
    return library().attn_status_string(int(status)).decode()


def _check(call, status):
    if status != CGQA_OK:
        detail = ""
        if status == CGQA_EHIP:
            detail = f"hipError {library().cgqa_last_hip_error()}"
        raise CgqaError(call, status, detail)


def _torch():
    import torch
    return torch


def _stream_ptr(stream):
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _need(t, name, dtype, shape, rows=False):
    """Checks a tensor's type, shape and device. With rows=True a [B, T, H, d] tensor may
    be a view whose tokens sit every rs elements (strides (T*rs, rs, d, 1), rs >= H*d);
    returns rs (H*d for a contiguous tensor)."""
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.is_contiguous():
        return shape[2] * shape[3] if rows else None
    if not rows:
        raise ValueError(f"{name} must be contiguous")
    B, T, H, d = shape
    st = t.stride()
    rs = st[1] if T > 1 else (st[0] if B > 1 else H * d)
    ok = st[3] == 1 and (H == 1 or st[2] == d) and (B == 1 or T == 1 or st[0] == T * st[1]) and rs >= H * d
    if not ok:
        raise ValueError(f"{name} must be [B, T, H, d] with strides (T*rs, rs, d, 1), got {st}")
    return rs


def _dims(q, k):
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q and k must be [B, T, H, d]")
    B, T, Hq, d = q.shape
    return B, T, Hq, k.shape[2], d


def _scale(scale, d):
    return float(1.0 / math.sqrt(d)) if scale is None else float(scale)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr())


def _kv_stride(rk, rv):
    if rk != rv:
        raise ValueError(f"k and v must share one row stride, got {rk} and {rv}")
    return rk


def attn_fwd(q, k, v, scale=None, o=None, lse=None, stream=None, rope=None):
    """o [B,T,Hq,d] bf16 and lse [B,Hq,T] fp32 for bf16 q [B,T,Hq,d], k, v [B,T,Hkv,d].
    q, k, v and o may be row-strided views (e.g. of one packed QKV buffer). With
    rope=(cos, sin) (fp32 [T, d/2]), q and k are the unrotated, contiguous tensors and are
    rotated as they are loaded (attn_fwd_rope, d = 64)."""
    torch = _torch()
    B, T, Hq, Hkv, d = _dims(q, k)
    rq = _need(q, "q", torch.bfloat16, (B, T, Hq, d), rows=True)
    rkv = _kv_stride(_need(k, "k", torch.bfloat16, (B, T, Hkv, d), rows=True),
                     _need(v, "v", torch.bfloat16, (B, T, Hkv, d), rows=True))
    if o is None:
        o = torch.empty((B, T, Hq, d), dtype=torch.bfloat16, device=q.device)
    if lse is None:
        lse = torch.empty((B, Hq, T), dtype=torch.float32, device=q.device)
    ro = _need(o, "o", torch.bfloat16, (B, T, Hq, d), rows=True)
    _need(lse, "lse", torch.float32, (B, Hq, T))
    lib = library()
    if rope is not None:
        if (rq, rkv, ro) != (Hq * d, Hkv * d, Hq * d):
            raise ValueError("attn_fwd with rope takes contiguous q, k, v and o")
        cos, sin = _rope_tables(rope, T, d)
        _check("attn_fwd_rope", lib.attn_fwd_rope(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(cos),
                                                  _ptr(sin), B, T, Hq, Hkv, d, _scale(scale, d),
                                                  _stream_ptr(stream)))
    elif (rq, rkv, ro) == (Hq * d, Hkv * d, Hq * d):
        _check("attn_fwd", lib.attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                                        B, T, Hq, Hkv, d, _scale(scale, d), _stream_ptr(stream)))
    else:
        _check("attn_fwd_strided", lib.attn_fwd_strided(
            _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, T, Hq, Hkv, d, rq, rkv, ro,
            _scale(scale, d), _stream_ptr(stream)))
    return o, lse


def _grad_code(dtype):
    torch = _torch()
    return CGQA_GRAD_BF16 if dtype == torch.bfloat16 else CGQA_GRAD_F32


def _rope_tables(rope, T, d):
    torch = _torch()
    cos, sin = rope
    for t, name in ((cos, "rope cos"), (sin, "rope sin")):
        _need(t.view(1, 1, *t.shape), name, torch.float32, (1, 1, T, d // 2))
    return cos, sin


def _absmax_layout(B, Hq, T):
    """(offset, count) in floats of the dO block maxima behind a delta of B*Hq*T floats
    (offset rounded up to 16 bytes)."""
    n = B * Hq * T
    return (n + 3) // 4 * 4, B * Hq * ((T + 31) // 32)


def bwd_delta(B, Hq, T, device=None):
    """The delta that attn_bwd_dq writes and attn_bwd_dkv reads: a [B, Hq, T] fp32 view at
    the start of an allocation that also holds the dO block maxima (B*Hq*ceil(T/32)
    floats, the dO_absmax workspace of the C calls) that carry the scale of dO from one
    call to the other."""
    torch = _torch()
    off, nm = _absmax_layout(B, Hq, T)
    buf = torch.empty(off + nm, dtype=torch.float32, device=device)
    return buf[:B * Hq * T].view(B, Hq, T)


def _absmax_ptr(delta, B, Hq, T):
    off, nm = _absmax_layout(B, Hq, T)
    if (delta.storage_offset() + off + nm) * 4 > delta.untyped_storage().nbytes():
        raise ValueError("delta must come from bwd_delta() or attn_bwd_dq (its allocation carries the dO maxima)")
    return ctypes.c_void_p(delta.data_ptr() + 4 * off)


def attn_bwd_dq(q, k, v, o, do, lse, scale=None, delta=None, dq=None, stream=None, grad_dtype=None, rope=None):
    """delta [B,Hq,T] fp32 and dq [B,T,Hq,d], fp32 or bf16 (the dtype of the dq given,
    else grad_dtype, else fp32). delta, if given, comes from bwd_delta(): its allocation
    also receives the dO block maxima for attn_bwd_dkv. Inputs and dq may be row-strided
    views. With
    rope=(cos, sin) (fp32 [T, d/2]), q and k are the rotated tensors and dq is returned
    with respect to the unrotated q (contiguous tensors, fp32 dq)."""
    torch = _torch()
    B, T, Hq, Hkv, d = _dims(q, k)
    rq, ro, rdo = (_need(t, name, torch.bfloat16, (B, T, Hq, d), rows=True)
                   for t, name in ((q, "q"), (o, "o"), (do, "do")))
    rkv = _kv_stride(_need(k, "k", torch.bfloat16, (B, T, Hkv, d), rows=True),
                     _need(v, "v", torch.bfloat16, (B, T, Hkv, d), rows=True))
    _need(lse, "lse", torch.float32, (B, Hq, T))
    if delta is None:
        delta = bwd_delta(B, Hq, T, device=q.device)
    if dq is None:
        dq = torch.empty((B, T, Hq, d), dtype=grad_dtype or torch.float32, device=q.device)
    _need(delta, "delta", torch.float32, (B, Hq, T))
    am = _absmax_ptr(delta, B, Hq, T)
    rdq = _need(dq, "dq", (torch.float32, torch.bfloat16), (B, T, Hq, d), rows=True)
    lib = library()
    contiguous = (rq, rkv, ro, rdo, rdq) == (Hq * d, Hkv * d, Hq * d, Hq * d, Hq * d)
    if rope is not None:
        if not contiguous or dq.dtype != torch.float32:
            raise ValueError("the rotary backward takes contiguous tensors and an fp32 dq")
        cos, sin = _rope_tables(rope, T, d)
        _check("attn_bwd_dq_rope", lib.attn_bwd_dq_rope(
            _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(do), _ptr(lse), _ptr(delta), am, _ptr(dq), _ptr(cos), _ptr(sin),
            B, T, Hq, Hkv, d, _scale(scale, d), _stream_ptr(stream)))
    elif contiguous and dq.dtype == torch.float32:
        _check("attn_bwd_dq", lib.attn_bwd_dq(
            _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(do), _ptr(lse), _ptr(delta), am, _ptr(dq),
            B, T, Hq, Hkv, d, _scale(scale, d), _stream_ptr(stream)))
    else:
        _check("attn_bwd_dq_strided", lib.attn_bwd_dq_strided(
            _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(do), _ptr(lse), _ptr(delta), am, _ptr(dq),
            B, T, Hq, Hkv, d, rq, rkv, ro, rdo, rdq, _grad_code(dq.dtype), _scale(scale, d), _stream_ptr(stream)))
    return delta, dq


def attn_bwd_dkv(q, k, v, do, lse, delta, scale=None, dk=None, dv=None, stream=None, grad_dtype=None, rope=None):
    """dk, dv [B,T,Hkv,d], fp32 or bf16 (the dtype of the dk/dv given, else grad_dtype,
    else fp32). Enqueue after attn_bwd_dq on the same stream, with the delta it returned
    (whose allocation carries the dO maxima). Inputs and dk, dv may be
    row-strided views (dk and dv with one row stride). With rope=(cos, sin), q and k are
    the rotated tensors and dk is returned with respect to the unrotated k (contiguous
    tensors, fp32 gradients)."""
    torch = _torch()
    B, T, Hq, Hkv, d = _dims(q, k)
    rq, rdo = (_need(t, name, torch.bfloat16, (B, T, Hq, d), rows=True) for t, name in ((q, "q"), (do, "do")))
    rkv = _kv_stride(_need(k, "k", torch.bfloat16, (B, T, Hkv, d), rows=True),
                     _need(v, "v", torch.bfloat16, (B, T, Hkv, d), rows=True))
    _need(lse, "lse", torch.float32, (B, Hq, T))
    _need(delta, "delta", torch.float32, (B, Hq, T))
    am = _absmax_ptr(delta, B, Hq, T)
    if dk is None:
        dk = torch.empty((B, T, Hkv, d), dtype=grad_dtype or torch.float32, device=q.device)
    if dv is None:
        dv = torch.empty((B, T, Hkv, d), dtype=dk.dtype, device=q.device)
    if dk.dtype != dv.dtype:
        raise TypeError(f"dk and dv must have one dtype, got {dk.dtype} and {dv.dtype}")
    rdk = _need(dk, "dk", (torch.float32, torch.bfloat16), (B, T, Hkv, d), rows=True)
    rdv = _need(dv, "dv", (torch.float32, torch.bfloat16), (B, T, Hkv, d), rows=True)
    if rdk != rdv:
        raise ValueError(f"dk and dv must share one row stride, got {rdk} and {rdv}")
    lib = library()
    contiguous = (rq, rkv, rdo, rdk) == (Hq * d, Hkv * d, Hq * d, Hkv * d)
    if rope is not None:
        if not contiguous or dk.dtype != torch.float32:
            raise ValueError("the rotary backward takes contiguous tensors and fp32 dk, dv")
        cos, sin = _rope_tables(rope, T, d)
        _check("attn_bwd_dkv_rope", lib.attn_bwd_dkv_rope(
            _ptr(q), _ptr(k), _ptr(v), _ptr(do), _ptr(lse), _ptr(delta), am, _ptr(dk), _ptr(dv), _ptr(cos), _ptr(sin),
            B, T, Hq, Hkv, d, _scale(scale, d), _stream_ptr(stream)))
    elif contiguous and dk.dtype == torch.float32:
        _check("attn_bwd_dkv", lib.attn_bwd_dkv(
            _ptr(q), _ptr(k), _ptr(v), _ptr(do), _ptr(lse), _ptr(delta), am, _ptr(dk), _ptr(dv),
            B, T, Hq, Hkv, d, _scale(scale, d), _stream_ptr(stream)))
    else:
        _check("attn_bwd_dkv_strided", lib.attn_bwd_dkv_strided(
            _ptr(q), _ptr(k), _ptr(v), _ptr(do), _ptr(lse), _ptr(delta), am, _ptr(dk), _ptr(dv),
            B, T, Hq, Hkv, d, rq, rkv, rdo, rdk, _grad_code(dk.dtype), _scale(scale, d), _stream_ptr(stream)))
    return dk, dv


def attn_naive_workspace_bytes(B, T, Hq):
    return int(library().attn_naive_workspace_bytes(int(B), int(T), int(Hq)))


def _workspace(B, T, Hq, workspace, device):
    torch = _torch()
    need = attn_naive_workspace_bytes(B, T, Hq)
    if workspace is None:
        workspace = torch.empty((max(need, 4) // 4,), dtype=torch.float32, device=device)
    if workspace.dtype != torch.float32 or not workspace.is_cuda or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous float32 device tensor")
    return workspace


def attn_naive_fwd(q, k, v, scale=None, o=None, lse=None, workspace=None, stream=None):
    """Naive attention (the GPU reference mode): o [B,T,Hq,d] bf16 and lse [B,Hq,T] fp32
    with every T x T probability stored in `workspace` (fp32, allocated if None).
    Contiguous tensors; 1 <= d <= 128."""
    torch = _torch()
    B, T, Hq, Hkv, d = _dims(q, k)
    _need(q, "q", torch.bfloat16, (B, T, Hq, d))
    _need(k, "k", torch.bfloat16, (B, T, Hkv, d))
    _need(v, "v", torch.bfloat16, (B, T, Hkv, d))
    if o is None:
        o = torch.empty((B, T, Hq, d), dtype=torch.bfloat16, device=q.device)
    if lse is None:
        lse = torch.empty((B, Hq, T), dtype=torch.float32, device=q.device)
    _need(o, "o", torch.bfloat16, (B, T, Hq, d))
    _need(lse, "lse", torch.float32, (B, Hq, T))
    ws = _workspace(B, T, Hq, workspace, q.device)
    _check("attn_naive_fwd", library().attn_naive_fwd(
        _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(ws), ws.numel() * 4,
        B, T, Hq, Hkv, d, _scale(scale, d), _stream_ptr(stream)))
    return o, lse


def attn_naive_bwd(q, k, v, do, scale=None, delta=None, dq=None, dk=None, dv=None, workspace=None,
                   stream=None):
    """Naive backward of L = sum(O * dO): delta [B,Hq,T], dq [B,T,Hq,d], dk, dv [B,T,Hkv,d],
    all fp32, recomputing the probabilities into `workspace`. Contiguous tensors."""
    torch = _torch()
    B, T, Hq, Hkv, d = _dims(q, k)
    _need(q, "q", torch.bfloat16, (B, T, Hq, d))
    _need(k, "k", torch.bfloat16, (B, T, Hkv, d))
    _need(v, "v", torch.bfloat16, (B, T, Hkv, d))
    _need(do, "do", torch.bfloat16, (B, T, Hq, d))
    f32 = dict(dtype=torch.float32, device=q.device)
    delta = torch.empty((B, Hq, T), **f32) if delta is None else delta
    dq = torch.empty((B, T, Hq, d), **f32) if dq is None else dq
    dk = torch.empty((B, T, Hkv, d), **f32) if dk is None else dk
    dv = torch.empty((B, T, Hkv, d), **f32) if dv is None else dv
    _need(delta, "delta", torch.float32, (B, Hq, T))
    _need(dq, "dq", torch.float32, (B, T, Hq, d))
    _need(dk, "dk", torch.float32, (B, T, Hkv, d))
    _need(dv, "dv", torch.float32, (B, T, Hkv, d))
    ws = _workspace(B, T, Hq, workspace, q.device)
    _check("attn_naive_bwd", library().attn_naive_bwd(
        _ptr(q), _ptr(k), _ptr(v), _ptr(do), _ptr(delta), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(ws),
        ws.numel() * 4, B, T, Hq, Hkv, d, _scale(scale, d), _stream_ptr(stream)))
    return delta, dq, dk, dv


def gemm_workspace_bytes(M, N, K):
    return int(library().cgqa_gemm_workspace_bytes(int(M), int(N), int(K)))


def gemm(a, b, r=None, c=None, a_km=False, b_kn=False, out_dtype=None, workspace=None, stream=None):
    """C = A B^T (+ R) on the matrix core. a: bf16 [M, K] (or [K, M] with a_km); b: bf16
    [N, K] (or [K, N] with b_kn); r: fp32 [M, N] or None (may be c itself); c: output
    [M, N], fp32 or bf16 (allocated with out_dtype, default fp32, if None); workspace:
    None or a contiguous fp32 device tensor for splitting long K (gemm_workspace_bytes)."""
    torch = _torch()
    if a.dim() != 2 or b.dim() != 2:
        raise ValueError("a and b must be 2-D")
    M, K = (a.shape[1], a.shape[0]) if a_km else (a.shape[0], a.shape[1])
    N, Kb = (b.shape[1], b.shape[0]) if b_kn else (b.shape[0], b.shape[1])
    if K != Kb:
        raise ValueError(f"inner sizes differ: {K} and {Kb}")
    _need4 = lambda t, name, dt, shape: _need(t.view(1, 1, *t.shape), name, dt, (1, 1) + tuple(shape))
    _need4(a, "a", torch.bfloat16, a.shape)
    _need4(b, "b", torch.bfloat16, b.shape)
    if c is None:
        c = torch.empty((M, N), dtype=out_dtype or torch.float32, device=a.device)
    _need4(c, "c", (torch.float32, torch.bfloat16), (M, N))
    if r is not None:
        _need4(r, "r", torch.float32, (M, N))
    flags = (CGQA_GEMM_A_KM if a_km else 0) | (CGQA_GEMM_B_KN if b_kn else 0) | \
        (CGQA_GEMM_C_BF16 if c.dtype == torch.bfloat16 else 0)
    ws, wsb = None, 0
    if workspace is not None:
        if workspace.dtype != torch.float32 or not workspace.is_cuda or not workspace.is_contiguous():
            raise ValueError("workspace must be a contiguous float32 device tensor")
        ws, wsb = _ptr(workspace), workspace.numel() * 4
    _check("cgqa_gemm", library().cgqa_gemm(_ptr(a), _ptr(b), _ptr(c), None if r is None else _ptr(r),
                                            M, N, K, flags, ws, wsb, _stream_ptr(stream)))
    return c


def rope_qk(q, k, cos, sin, q_out=None, k_out=None, stream=None):
    """Rotary embedding of bf16 q [B,T,Hq,d] and k [B,T,Hkv,d] with fp32 tables cos, sin
    [T, d/2]: returns (q_out, k_out), bf16. Tensors may be row-strided views; q_out=q and
    k_out=k rotate in place (e.g. inside a packed QKV buffer)."""
    torch = _torch()
    B, T, Hq, Hkv, d = _dims(q, k)
    rq = _need(q, "q", torch.bfloat16, (B, T, Hq, d), rows=True)
    rk = _need(k, "k", torch.bfloat16, (B, T, Hkv, d), rows=True)
    if q_out is None:
        q_out = torch.empty((B, T, Hq, d), dtype=torch.bfloat16, device=q.device)
    if k_out is None:
        k_out = torch.empty((B, T, Hkv, d), dtype=torch.bfloat16, device=q.device)
    rqo = _need(q_out, "q_out", torch.bfloat16, (B, T, Hq, d), rows=True)
    rko = _need(k_out, "k_out", torch.bfloat16, (B, T, Hkv, d), rows=True)
    cos, sin = _rope_tables((cos, sin), T, d)
    _check("attn_rope_qk", library().attn_rope_qk(
        _ptr(q), _ptr(k), _ptr(q_out), _ptr(k_out), _ptr(cos), _ptr(sin), B, T, Hq, Hkv, d,
        rq, rk, rqo, rko, _stream_ptr(stream)))
    return q_out, k_out


def calib_mfma(blocks, iters, stream=None, sink=None, clocks=None):
    """Launches the matrix-core calibration (cgqa_calib_mfma): returns the device sink
    (blocks*256 fp32, each iters/64), the device clocks (int64 [2]: block 0's loop in shader
    clocks and in 100 MHz ticks) and the launch's flop count. sink and clocks may be given
    (to launch without allocating)."""
    torch = _torch()
    if sink is None:
        sink = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
    if clocks is None:
        clocks = torch.zeros(2, dtype=torch.int64, device="cuda")
    _need(sink, "sink", torch.float32, (blocks * 256,))
    _need(clocks, "clocks", torch.int64, (2,))
    flops = ctypes.c_double(0.0)
    _check("cgqa_calib_mfma", library().cgqa_calib_mfma(_ptr(sink), _ptr(clocks), blocks, iters,
                                                        ctypes.byref(flops), _stream_ptr(stream)))
    return sink, clocks, flops.value

