// C-ABI entry points: argument validation (before any HIP call) and kernel dispatch.
// The operations and their contracts are stated in include/cgqa.h.
#include <math.h>
#include <stdint.h>

#include "../../include/cgqa.h"
#include "cgqa_launch.hpp"

namespace {

thread_local int g_last_hip_error = 0;

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// A tensor as the kernels address it: `rows` rows (B*T tokens) of `width` elements
// (H*d) every `rs` elements, `eb` bytes per element.
struct View {
    const void* p;
    int64_t rows, width, rs, eb;
    uintptr_t lo() const { return (uintptr_t)p; }
    uintptr_t hi() const { return (uintptr_t)p + (uintptr_t)(((rows - 1) * rs + width) * eb); }
};

// True if no element of a lies in b. Tensors whose byte ranges meet must have the same
// row pitch and column windows that do not intersect within a row (interleaved heads of
// one packed buffer); any other meeting ranges count as overlapping.
bool disjoint(View a, View b) {
    if (a.hi() <= b.lo() || b.hi() <= a.lo()) return true;
    if (a.rs * a.eb != b.rs * b.eb) return false;
    if (a.lo() > b.lo()) {
        View t = a;
        a = b;
        b = t;
    }
    const uint64_t pitch = (uint64_t)(a.rs * a.eb);
    const uint64_t k = (uint64_t)(b.lo() - a.lo()) % pitch;   // b's first byte within a row of a
    return k >= (uint64_t)(a.width * a.eb) && k + (uint64_t)(b.width * b.eb) <= pitch;
}

// Shape checks shared by the calls. Returns CGQA_OK, or sets *empty for B or T = 0.
// The flash kernels take d = 64 or 128, the naive ones any d from 1 to 128.
int check_shape(int B, int T, int Hq, int Hkv, int d, float scale, bool* empty, bool naive = false) {
    *empty = false;
    if (B < 0 || T < 0 || Hq < 1 || Hkv < 1) return CGQA_EINVAL;
    if (Hq % Hkv != 0) return CGQA_EINVAL;
    if (!(scale > 0.0f) || !isfinite(scale)) return CGQA_EINVAL;
    if (naive ? (d < 1 || d > 128) : (d != 64 && d != 128)) return CGQA_EUNSUPPORTED;
    if ((int64_t)B * Hq * T >= ((int64_t)1 << 31)) return CGQA_EINVAL;
    if (B == 0 || T == 0) *empty = true;
    return CGQA_OK;
}

// A row stride of a tensor with `width` elements per row: at least the row, at most
// 2^31 elements in all (kernel offsets are 32-bit within a tensor's rows), and a
// multiple of `align` elements (whole 16- or 8-byte accesses).
int check_stride(int64_t rs, int64_t width, int64_t rows, int64_t align) {
    if (rs < width || rows * rs >= ((int64_t)1 << 31)) return CGQA_EINVAL;
    if (rs % align != 0) return CGQA_EUNSUPPORTED;
    return CGQA_OK;
}

int finish(hipError_t e) {
    if (e != hipSuccess) {
        g_last_hip_error = (int)e;
        return CGQA_EHIP;
    }
    return CGQA_OK;
}

int fwd_impl(const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* o, float* lse,
             int B, int T, int Hq, int Hkv, int d, int q_rs, int kv_rs, int o_rs, float scale, void* stream,
             bool rope = false, const float* rope_cos = nullptr, const float* rope_sin = nullptr) {
    bool empty = false;
    int rc = check_shape(B, T, Hq, Hkv, d, scale, &empty);
    if (rc != CGQA_OK) return rc;
    if (rope && d != 64) return CGQA_EUNSUPPORTED;
    const int64_t rows = (int64_t)B * T, wq = (int64_t)Hq * d, wkv = (int64_t)Hkv * d;
    const int64_t rcs[3] = {check_stride(q_rs, wq, rows, 8), check_stride(kv_rs, wkv, rows, 8),
                            check_stride(o_rs, wq, rows, 4)};
    for (int64_t r : rcs)
        if (r == CGQA_EINVAL) return CGQA_EINVAL;
    for (int64_t r : rcs)
        if (r != CGQA_OK) return (int)r;
    if (empty) return CGQA_OK;
    if (!q || !k || !v || !o || !lse) return CGQA_EINVAL;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse))
        return CGQA_EUNSUPPORTED;
    const View vo{o, rows, wq, o_rs, 2}, vl{lse, 1, (int64_t)B * Hq * T, (int64_t)B * Hq * T, 4};
    const View ins[3] = {View{q, rows, wq, q_rs, 2}, View{k, rows, wkv, kv_rs, 2}, View{v, rows, wkv, kv_rs, 2}};
    if (!disjoint(vo, vl)) return CGQA_EINVAL;
    for (const View& s : ins)
        if (!disjoint(s, vo) || !disjoint(s, vl)) return CGQA_EINVAL;
    if (rope) {
        if (!rope_cos || !rope_sin) return CGQA_EINVAL;
        if (!aligned16(rope_cos) || !aligned16(rope_sin)) return CGQA_EUNSUPPORTED;
        const int64_t nt = (int64_t)T * (d / 2);
        const View vc{rope_cos, 1, nt, nt, 4}, vs{rope_sin, 1, nt, nt, 4};
        if (!disjoint(vc, vo) || !disjoint(vc, vl) || !disjoint(vs, vo) || !disjoint(vs, vl)) return CGQA_EINVAL;
    }

    cgqa::FwdArgs a{};
    a.q = q; a.k = k; a.v = v; a.o = o; a.lse = lse;
    a.B = B; a.T = T; a.Hq = Hq; a.Hkv = Hkv; a.d = d;
    a.q_rs = q_rs; a.kv_rs = kv_rs; a.o_rs = o_rs;
    a.scale_log2 = (float)((double)scale * 1.4426950408889634);
    a.div = cgqa::make_map_divs(B, Hq, Hkv);
    if (rope) {
        a.rope_cos = rope_cos;
        a.rope_sin = rope_sin;
        return finish(cgqa::launch_fwd_rope(a, (hipStream_t)stream));
    }
    return finish(cgqa::launch_fwd(a, (hipStream_t)stream));
}

struct BwdStrides {
    int q_rs, kv_rs, o_rs, do_rs, dq_rs, dkv_rs, grad;
};

int bwd_impl(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* o,
             const uint16_t* dO, const float* lse, const float* delta_in, float* delta_out,
             const float* absmax_in, float* absmax_out, void* dq, void* dk, void* dv, int B, int T, int Hq, int Hkv, int d, const BwdStrides& st,
             float scale, void* stream, bool is_dq, const float* rope_cos = nullptr,
             const float* rope_sin = nullptr) {
    bool empty = false;
    int rc = check_shape(B, T, Hq, Hkv, d, scale, &empty);
    if (rc != CGQA_OK) return rc;
    if (st.grad != CGQA_GRAD_F32 && st.grad != CGQA_GRAD_BF16) return CGQA_EINVAL;
    const int64_t rows = (int64_t)B * T, wq = (int64_t)Hq * d, wkv = (int64_t)Hkv * d, nr = (int64_t)B * Hq * T;
    const int64_t nm = (int64_t)B * Hq * ((T + 31) / 32);   // dO block maxima
    const int64_t geb = st.grad == CGQA_GRAD_BF16 ? 2 : 4;
    int64_t rcs[4] = {check_stride(st.q_rs, wq, rows, 8), check_stride(st.kv_rs, wkv, rows, 8),
                      check_stride(st.do_rs, wq, rows, 8),
                      is_dq ? check_stride(st.dq_rs, wq, rows, 4) : check_stride(st.dkv_rs, wkv, rows, 4)};
    const int64_t rco = is_dq ? check_stride(st.o_rs, wq, rows, 8) : CGQA_OK;
    for (int64_t r : rcs)
        if (r == CGQA_EINVAL) return CGQA_EINVAL;
    if (rco == CGQA_EINVAL) return CGQA_EINVAL;
    for (int64_t r : rcs)
        if (r != CGQA_OK) return (int)r;
    if (rco != CGQA_OK) return (int)rco;
    if (empty) return CGQA_OK;
    const View vq{q, rows, wq, st.q_rs, 2}, vk{k, rows, wkv, st.kv_rs, 2}, vv{v, rows, wkv, st.kv_rs, 2},
        vdo{dO, rows, wq, st.do_rs, 2}, vl{lse, 1, nr, nr, 4};
    if (is_dq) {
        if (!q || !k || !v || !o || !dO || !lse || !delta_out || !absmax_out || !dq) return CGQA_EINVAL;
        if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(dO) ||
            !aligned16(lse) || !aligned16(delta_out) || !aligned16(absmax_out) || !aligned16(dq))
            return CGQA_EUNSUPPORTED;
        const View outs[3] = {View{delta_out, 1, nr, nr, 4}, View{dq, rows, wq, st.dq_rs, geb},
                              View{absmax_out, 1, nm, nm, 4}};
        const View ins[6] = {vq, vk, vv, View{o, rows, wq, st.o_rs, 2}, vdo, vl};
        for (int x = 0; x < 3; ++x)
            for (int y = x + 1; y < 3; ++y)
                if (!disjoint(outs[x], outs[y])) return CGQA_EINVAL;
        for (const View& s : ins)
            for (const View& t : outs)
                if (!disjoint(s, t)) return CGQA_EINVAL;
    } else {
        if (!q || !k || !v || !dO || !lse || !delta_in || !absmax_in || !dk || !dv) return CGQA_EINVAL;
        if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(dO) || !aligned16(lse) ||
            !aligned16(delta_in) || !aligned16(absmax_in) || !aligned16(dk) || !aligned16(dv))
            return CGQA_EUNSUPPORTED;
        const View outs[2] = {View{dk, rows, wkv, st.dkv_rs, geb}, View{dv, rows, wkv, st.dkv_rs, geb}};
        const View ins[7] = {vq, vk, vv, vdo, vl, View{delta_in, 1, nr, nr, 4}, View{absmax_in, 1, nm, nm, 4}};
        if (!disjoint(outs[0], outs[1])) return CGQA_EINVAL;
        for (const View& s : ins)
            if (!disjoint(s, outs[0]) || !disjoint(s, outs[1])) return CGQA_EINVAL;
    }
    if (rope_cos || rope_sin) {
        if (!rope_cos || !rope_sin) return CGQA_EINVAL;
        if (!aligned16(rope_cos) || !aligned16(rope_sin)) return CGQA_EUNSUPPORTED;
        const int64_t nt = (int64_t)T * (d / 2);
        const View vc{rope_cos, 1, nt, nt, 4}, vs{rope_sin, 1, nt, nt, 4};
        const View outs[3] = {is_dq ? View{delta_out, 1, nr, nr, 4} : View{dk, rows, wkv, st.dkv_rs, geb},
                              is_dq ? View{dq, rows, wq, st.dq_rs, geb} : View{dv, rows, wkv, st.dkv_rs, geb},
                              is_dq ? View{absmax_out, 1, nm, nm, 4} : View{dv, rows, wkv, st.dkv_rs, geb}};
        for (int x = 0; x < 3; ++x)
            if (!disjoint(outs[x], vc) || !disjoint(outs[x], vs)) return CGQA_EINVAL;
    }
    cgqa::BwdArgs a{};
    a.q = q; a.k = k; a.v = v; a.o = o; a.dO = dO; a.lse = lse;
    a.rope_cos = rope_cos; a.rope_sin = rope_sin;
    a.delta = is_dq ? delta_out : const_cast<float*>(delta_in);
    a.do_absmax = is_dq ? absmax_out : const_cast<float*>(absmax_in);
    a.dq = dq; a.dk = dk; a.dv = dv;
    a.B = B; a.T = T; a.Hq = Hq; a.Hkv = Hkv; a.d = d;
    a.q_rs = st.q_rs; a.kv_rs = st.kv_rs; a.o_rs = st.o_rs; a.do_rs = st.do_rs;
    a.dq_rs = st.dq_rs; a.dkv_rs = st.dkv_rs; a.grad_bf16 = st.grad == CGQA_GRAD_BF16 ? 1 : 0;
    a.scale = scale;
    a.scale_log2 = (float)((double)scale * 1.4426950408889634);
    a.div = cgqa::make_map_divs(B, Hq, Hkv);
    return finish(is_dq ? cgqa::launch_bwd_dq(a, (hipStream_t)stream)
                        : cgqa::launch_bwd_dkv(a, (hipStream_t)stream));
}

// Bytes of the naive workspace, or -1 for sizes no call accepts.
int64_t naive_ws_bytes(int B, int T, int Hq) {
    if (B < 0 || T < 0 || Hq < 1 || (int64_t)B * Hq * T >= ((int64_t)1 << 31)) return -1;
    return (int64_t)B * Hq * T * T * 4;
}

// Both naive calls: contiguous tensors, an fp32 workspace of B*Hq*T*T floats that
// overlaps nothing else. Inputs in[0..nin), outputs out[0..nout) as byte views.
int naive_impl(bool fwd, const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* dO,
               uint16_t* o, float* lse, float* delta, float* dq, float* dk, float* dv, float* ws,
               size_t ws_bytes, int B, int T, int Hq, int Hkv, int d, float scale, void* stream) {
    bool empty = false;
    int rc = check_shape(B, T, Hq, Hkv, d, scale, &empty, true);
    if (rc != CGQA_OK) return rc;
    const int64_t rows = (int64_t)B * T, wq = (int64_t)Hq * d, wkv = (int64_t)Hkv * d, nr = (int64_t)B * Hq * T;
    if (rows * wq >= ((int64_t)1 << 31)) return CGQA_EINVAL;
    if (empty) return CGQA_OK;
    const int64_t need = naive_ws_bytes(B, T, Hq);
    if (!ws || (uint64_t)ws_bytes < (uint64_t)need) return CGQA_EINVAL;
    const View vq{q, rows, wq, wq, 2}, vk{k, rows, wkv, wkv, 2}, vv{v, rows, wkv, wkv, 2},
        vw{ws, 1, need / 4, need / 4, 4};
    if (fwd) {
        if (!q || !k || !v || !o || !lse) return CGQA_EINVAL;
        if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse) || !aligned16(ws))
            return CGQA_EUNSUPPORTED;
        const View outs[3] = {View{o, rows, wq, wq, 2}, View{lse, 1, nr, nr, 4}, vw};
        const View ins[3] = {vq, vk, vv};
        for (int x = 0; x < 3; ++x) {
            for (int y = x + 1; y < 3; ++y)
                if (!disjoint(outs[x], outs[y])) return CGQA_EINVAL;
            for (const View& s : ins)
                if (!disjoint(s, outs[x])) return CGQA_EINVAL;
        }
    } else {
        if (!q || !k || !v || !dO || !delta || !dq || !dk || !dv) return CGQA_EINVAL;
        if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(dO) || !aligned16(delta) ||
            !aligned16(dq) || !aligned16(dk) || !aligned16(dv) || !aligned16(ws))
            return CGQA_EUNSUPPORTED;
        const View outs[5] = {View{delta, 1, nr, nr, 4}, View{dq, rows, wq, wq, 4}, View{dk, rows, wkv, wkv, 4},
                              View{dv, rows, wkv, wkv, 4}, vw};
        const View ins[4] = {vq, vk, vv, View{dO, rows, wq, wq, 2}};
        for (int x = 0; x < 5; ++x) {
            for (int y = x + 1; y < 5; ++y)
                if (!disjoint(outs[x], outs[y])) return CGQA_EINVAL;
            for (const View& s : ins)
                if (!disjoint(s, outs[x])) return CGQA_EINVAL;
        }
    }
    cgqa::NaiveArgs a{};
    a.q = q; a.k = k; a.v = v; a.dO = dO; a.o = o; a.lse = lse; a.delta = delta;
    a.dq = dq; a.dk = dk; a.dv = dv; a.p = ws;
    a.B = B; a.T = T; a.Hq = Hq; a.Hkv = Hkv; a.d = d; a.scale = scale;
    return finish(fwd ? cgqa::launch_naive_fwd(a, (hipStream_t)stream) : cgqa::launch_naive_bwd(a, (hipStream_t)stream));
}

// use_scratch: the split-K partials go to the library's static per-device scratch
// (cgqa_gemm_static) instead of `ws`; shapes whose split needs more are rejected.
int gemm_impl(const uint16_t* A, const uint16_t* B, void* C, const float* R, int M, int N, int K, int flags,
              float* ws, size_t ws_bytes, void* stream, bool use_scratch = false) {
    if (M < 0 || N < 0 || K < 0) return CGQA_EINVAL;
    if (flags & ~(CGQA_GEMM_A_KM | CGQA_GEMM_B_KN | CGQA_GEMM_C_BF16)) return CGQA_EINVAL;
    const bool akm = flags & CGQA_GEMM_A_KM, bkn = flags & CGQA_GEMM_B_KN, cbf = flags & CGQA_GEMM_C_BF16;
    const int64_t lim = (int64_t)1 << 31;
    if ((int64_t)M * K >= lim || (int64_t)N * K >= lim || (int64_t)M * N >= lim) return CGQA_EINVAL;
    if (K % 32 != 0 || (akm && M % 8 != 0) || (bkn && N % 8 != 0)) return CGQA_EUNSUPPORTED;
    if (M == 0 || N == 0) return CGQA_OK;
    if (!C || (K > 0 && (!A || !B))) return CGQA_EINVAL;   // K == 0 reads neither A nor B
    if (!aligned16(A) || !aligned16(B) || !aligned16(C) || (R && !aligned16(R))) return CGQA_EUNSUPPORTED;
    if (R && cbf && (const void*)R == C) return CGQA_EINVAL;   // R = C only for an fp32 C
    const int64_t ceb = cbf ? 2 : 4;
    const View vc{C, 1, (int64_t)M * N, (int64_t)M * N, ceb};
    const View va{A, 1, (int64_t)M * K, (int64_t)M * K, 2}, vb{B, 1, (int64_t)N * K, (int64_t)N * K, 2};
    if (!disjoint(vc, va) || !disjoint(vc, vb)) return CGQA_EINVAL;
    if (R && (const void*)R != C && !disjoint(vc, View{R, 1, (int64_t)M * N, (int64_t)M * N, 4})) return CGQA_EINVAL;
    size_t need = 0;
    if (use_scratch) {
        need = (size_t)cgqa::gemm_splits(M, N, K, (size_t)-1);
        need = need > 1 ? need * cgqa::gemm_slice_floats(M, N) * 4 : 0;
        if (need > cgqa::kGemmScratchBytes) return CGQA_EINVAL;
    }
    if (ws) {
        if (!aligned16(ws)) return CGQA_EUNSUPPORTED;
        const int64_t n = (int64_t)(ws_bytes / 4);
        const View vw{ws, 1, n > 0 ? n : 1, n > 0 ? n : 1, 4};
        if (!disjoint(vw, vc) || (K > 0 && (!disjoint(vw, va) || !disjoint(vw, vb))) ||
            (R && !disjoint(vw, View{R, 1, (int64_t)M * N, (int64_t)M * N, 4})))
            return CGQA_EINVAL;
    }
    cgqa::GemmArgs a{};
    a.a = A; a.b = B; a.c = C; a.r = R;
    a.M = M; a.N = N; a.K = K;
    a.a_km = akm; a.b_kn = bkn; a.c_bf16 = cbf;
    a.ws = ws; a.ws_bytes = ws ? ws_bytes : 0;
    if (use_scratch && need > 0) {
        float* p = nullptr;
        const hipError_t e = cgqa::gemm_scratch(&p);
        if (e != hipSuccess) return finish(e);
        a.ws = p;
        a.ws_bytes = need;
    }
    return finish(cgqa::launch_gemm(a, (hipStream_t)stream));
}

}  // namespace

extern "C" {

int attn_rope_qk(const uint16_t* q, const uint16_t* k, uint16_t* q_out, uint16_t* k_out, const float* cos_t,
                 const float* sin_t, int B, int T, int Hq, int Hkv, int d, int q_row_stride, int k_row_stride,
                 int q_out_row_stride, int k_out_row_stride, void* stream) {
    bool empty = false;
    int rc = check_shape(B, T, Hq, Hkv, d, 1.0f, &empty);
    if (rc != CGQA_OK) return rc;
    const int64_t rows = (int64_t)B * T, wq = (int64_t)Hq * d, wk = (int64_t)Hkv * d;
    const int64_t rcs[4] = {check_stride(q_row_stride, wq, rows, 8), check_stride(k_row_stride, wk, rows, 8),
                            check_stride(q_out_row_stride, wq, rows, 8), check_stride(k_out_row_stride, wk, rows, 8)};
    for (int64_t r : rcs)
        if (r == CGQA_EINVAL) return CGQA_EINVAL;
    for (int64_t r : rcs)
        if (r != CGQA_OK) return (int)r;
    if (empty) return CGQA_OK;
    if (!q || !k || !q_out || !k_out || !cos_t || !sin_t) return CGQA_EINVAL;
    if (!aligned16(q) || !aligned16(k) || !aligned16(q_out) || !aligned16(k_out) || !aligned16(cos_t) ||
        !aligned16(sin_t))
        return CGQA_EUNSUPPORTED;
    const int64_t nt = (int64_t)T * (d / 2);
    const View vq{q, rows, wq, q_row_stride, 2}, vk{k, rows, wk, k_row_stride, 2},
        vqo{q_out, rows, wq, q_out_row_stride, 2}, vko{k_out, rows, wk, k_out_row_stride, 2},
        vc{cos_t, 1, nt, nt, 4}, vs{sin_t, 1, nt, nt, 4};
    // An output may be its own input exactly (in place); otherwise nothing may overlap it.
    const bool q_inplace = q_out == q && q_out_row_stride == q_row_stride;
    const bool k_inplace = k_out == k && k_out_row_stride == k_row_stride;
    if (!disjoint(vqo, vko) || !disjoint(vqo, vk) || !disjoint(vko, vq)) return CGQA_EINVAL;
    if ((!q_inplace && !disjoint(vqo, vq)) || (!k_inplace && !disjoint(vko, vk))) return CGQA_EINVAL;
    for (const View& o : {vqo, vko})
        if (!disjoint(o, vc) || !disjoint(o, vs)) return CGQA_EINVAL;
    cgqa::RopeArgs a{};
    a.q = q; a.k = k; a.q_out = q_out; a.k_out = k_out; a.cos = cos_t; a.sin = sin_t;
    a.B = B; a.T = T; a.Hq = Hq; a.Hkv = Hkv; a.d = d;
    a.q_rs = q_row_stride; a.k_rs = k_row_stride; a.qo_rs = q_out_row_stride; a.ko_rs = k_out_row_stride;
    return finish(cgqa::launch_rope(a, (hipStream_t)stream));
}

int attn_bwd_dq_rope(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* o,
                     const uint16_t* dO, const float* lse, float* delta, float* dO_absmax, float* dq,
                     const float* rope_cos,
                     const float* rope_sin, int B, int T, int Hq, int Hkv, int d, float scale, void* stream) {
    const int64_t wq = (int64_t)Hq * d, wkv = (int64_t)Hkv * d;
    if (Hq < 1 || Hkv < 1 || wq >= ((int64_t)1 << 31)) return CGQA_EINVAL;
    if (!rope_cos || !rope_sin) return CGQA_EINVAL;
    const BwdStrides st{(int)wq, (int)wkv, (int)wq, (int)wq, (int)wq, (int)wkv, CGQA_GRAD_F32};
    return bwd_impl(q, k, v, o, dO, lse, nullptr, delta, nullptr, dO_absmax, dq, nullptr, nullptr, B, T, Hq, Hkv, d, st, scale,
                    stream, true, rope_cos, rope_sin);
}

int attn_bwd_dkv_rope(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* dO,
                      const float* lse, const float* delta, const float* dO_absmax, float* dk, float* dv,
                      const float* rope_cos,
                      const float* rope_sin, int B, int T, int Hq, int Hkv, int d, float scale, void* stream) {
    const int64_t wq = (int64_t)Hq * d, wkv = (int64_t)Hkv * d;
    if (Hq < 1 || Hkv < 1 || wq >= ((int64_t)1 << 31)) return CGQA_EINVAL;
    if (!rope_cos || !rope_sin) return CGQA_EINVAL;
    const BwdStrides st{(int)wq, (int)wkv, (int)wq, (int)wq, (int)wq, (int)wkv, CGQA_GRAD_F32};
    return bwd_impl(q, k, v, nullptr, dO, lse, delta, nullptr, dO_absmax, nullptr, nullptr, dk, dv, B, T, Hq, Hkv, d, st, scale,
                    stream, false, rope_cos, rope_sin);
}

size_t cgqa_gemm_workspace_bytes(int M, int N, int K) {
    if (M <= 0 || N <= 0 || K <= 0 || K % 32 != 0 || (int64_t)M * N >= ((int64_t)1 << 31)) return 0;
    const int s = cgqa::gemm_splits(M, N, K, (size_t)-1);
    return s > 1 ? (size_t)s * cgqa::gemm_slice_floats(M, N) * 4 : 0;
}

int cgqa_gemm(const uint16_t* A, const uint16_t* B, void* C, const float* R, int M, int N, int K, int flags,
              float* workspace, size_t workspace_bytes, void* stream) {
    return gemm_impl(A, B, C, R, M, N, K, flags, workspace, workspace_bytes, stream);
}

int cgqa_calib_mfma(float* sink, uint64_t* clocks, int blocks, int iters, double* flops, void* stream) {
    if (blocks < 1 || blocks > (1 << 16) || iters < 1 || iters > (1 << 20)) return CGQA_EINVAL;
    if (!sink) return CGQA_EINVAL;
    if (!aligned16(sink) || (clocks && !aligned16(clocks))) return CGQA_EUNSUPPORTED;
    if (clocks) {
        const int64_t n = (int64_t)blocks * cgqa::kCalibThreads;
        if (!disjoint(View{sink, 1, n, n, 4}, View{clocks, 1, 2, 2, 8})) return CGQA_EINVAL;
    }
    if (flops) *flops = cgqa::calib_mfma_flops(blocks, iters);
    return finish(cgqa::launch_calib_mfma(sink, reinterpret_cast<unsigned long long*>(clocks), blocks, iters,
                                          (hipStream_t)stream));
}

static_assert(cgqa::kGemmScratchBytes == CGQA_GEMM_STATIC_SCRATCH_BYTES, "scratch size");

int cgqa_gemm_static(const uint16_t* A, const uint16_t* B, void* C, const float* R, int M, int N, int K,
                     int flags, void* stream) {
    return gemm_impl(A, B, C, R, M, N, K, flags, nullptr, 0, stream, true);
}

size_t attn_naive_workspace_bytes(int B, int T, int Hq) {
    const int64_t n = naive_ws_bytes(B, T, Hq);
    return n < 0 ? 0 : (size_t)n;
}

int attn_naive_fwd(const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* o, float* lse,
                   float* workspace, size_t workspace_bytes, int B, int T, int Hq, int Hkv, int d,
                   float scale, void* stream) {
    return naive_impl(true, q, k, v, nullptr, o, lse, nullptr, nullptr, nullptr, nullptr, workspace,
                      workspace_bytes, B, T, Hq, Hkv, d, scale, stream);
}

int attn_naive_bwd(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* dO,
                   float* delta, float* dq, float* dk, float* dv, float* workspace, size_t workspace_bytes,
                   int B, int T, int Hq, int Hkv, int d, float scale, void* stream) {
    return naive_impl(false, q, k, v, dO, nullptr, nullptr, delta, dq, dk, dv, workspace, workspace_bytes,
                      B, T, Hq, Hkv, d, scale, stream);
}

int attn_fwd(const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* o, float* lse,
             int B, int T, int Hq, int Hkv, int d, float scale, void* stream) {
    // Contiguous strides; a product that overflows int is caught by the shape check.
    const int64_t wq = (int64_t)Hq * d, wkv = (int64_t)Hkv * d;
    if (Hq < 1 || Hkv < 1 || wq >= ((int64_t)1 << 31)) return CGQA_EINVAL;
    return fwd_impl(q, k, v, o, lse, B, T, Hq, Hkv, d, (int)wq, (int)wkv, (int)wq, scale, stream);
}

int attn_fwd_rope(const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* o, float* lse,
                  const float* rope_cos, const float* rope_sin, int B, int T, int Hq, int Hkv, int d,
                  float scale, void* stream) {
    const int64_t wq = (int64_t)Hq * d, wkv = (int64_t)Hkv * d;
    if (Hq < 1 || Hkv < 1 || wq >= ((int64_t)1 << 31)) return CGQA_EINVAL;
    return fwd_impl(q, k, v, o, lse, B, T, Hq, Hkv, d, (int)wq, (int)wkv, (int)wq, scale, stream,
                    true, rope_cos, rope_sin);
}

int attn_fwd_strided(const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* o, float* lse,
                     int B, int T, int Hq, int Hkv, int d, int q_row_stride, int kv_row_stride,
                     int o_row_stride, float scale, void* stream) {
    return fwd_impl(q, k, v, o, lse, B, T, Hq, Hkv, d, q_row_stride, kv_row_stride, o_row_stride, scale, stream);
}

int attn_bwd_dq(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* o,
                const uint16_t* dO, const float* lse, float* delta, float* dO_absmax, float* dq,
                int B, int T, int Hq, int Hkv, int d, float scale, void* stream) {
    const int64_t wq = (int64_t)Hq * d, wkv = (int64_t)Hkv * d;
    if (Hq < 1 || Hkv < 1 || wq >= ((int64_t)1 << 31)) return CGQA_EINVAL;
    const BwdStrides st{(int)wq, (int)wkv, (int)wq, (int)wq, (int)wq, (int)wkv, CGQA_GRAD_F32};
    return bwd_impl(q, k, v, o, dO, lse, nullptr, delta, nullptr, dO_absmax, dq, nullptr, nullptr, B, T, Hq, Hkv, d, st, scale,
                    stream, true);
}

int attn_bwd_dkv(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* dO,
                 const float* lse, const float* delta, const float* dO_absmax, float* dk, float* dv,
                 int B, int T, int Hq, int Hkv, int d, float scale, void* stream) {
    const int64_t wq = (int64_t)Hq * d, wkv = (int64_t)Hkv * d;
    if (Hq < 1 || Hkv < 1 || wq >= ((int64_t)1 << 31)) return CGQA_EINVAL;
    const BwdStrides st{(int)wq, (int)wkv, (int)wq, (int)wq, (int)wq, (int)wkv, CGQA_GRAD_F32};
    return bwd_impl(q, k, v, nullptr, dO, lse, delta, nullptr, dO_absmax, nullptr, nullptr, dk, dv, B, T, Hq, Hkv, d, st, scale,
                    stream, false);
}

int attn_bwd_dq_strided(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* o,
                        const uint16_t* dO, const float* lse, float* delta, float* dO_absmax, void* dq,
                        int B, int T, int Hq, int Hkv, int d, int q_row_stride, int kv_row_stride,
                        int o_row_stride, int do_row_stride, int dq_row_stride, int grad_dtype,
                        float scale, void* stream) {
    const BwdStrides st{q_row_stride, kv_row_stride, o_row_stride, do_row_stride, dq_row_stride, 0, grad_dtype};
    return bwd_impl(q, k, v, o, dO, lse, nullptr, delta, nullptr, dO_absmax, dq, nullptr, nullptr, B, T, Hq, Hkv, d, st, scale,
                    stream, true);
}

int attn_bwd_dkv_strided(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* dO,
                         const float* lse, const float* delta, const float* dO_absmax, void* dk, void* dv,
                         int B, int T, int Hq, int Hkv, int d, int q_row_stride, int kv_row_stride,
                         int do_row_stride, int dkv_row_stride, int grad_dtype, float scale, void* stream) {
    const BwdStrides st{q_row_stride, kv_row_stride, 0, do_row_stride, 0, dkv_row_stride, grad_dtype};
    return bwd_impl(q, k, v, nullptr, dO, lse, delta, nullptr, dO_absmax, nullptr, nullptr, dk, dv, B, T, Hq, Hkv, d, st, scale,
                    stream, false);
}

const char* attn_status_string(int status) {
    switch (status) {
        case CGQA_OK: return "ok";
        case CGQA_EINVAL: return "invalid argument (null pointer, bad size, bad scale, overlap or too large)";
        case CGQA_EUNSUPPORTED: return "unsupported (head dim not 64 or 128, or pointer not 16-byte aligned)";
        case CGQA_EHIP: return "HIP runtime refused the kernel launch (see cgqa_last_hip_error)";
        default: return "unknown status";
    }
}

int cgqa_last_hip_error(void) { return g_last_hip_error; }

}  // extern "C"
