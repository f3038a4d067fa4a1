// C-ABI entry points: argument validation (before any HIP call) and kernel dispatch.
// The operations and their contracts are stated in include/cgqa.h.
#include <math.h>
#include <stdint.h>

#include "../../include/cgqa.h"
#include "cgqa_launch.hpp"

namespace {

thread_local int g_last_hip_error = 0;

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

struct Span {
    uintptr_t lo, hi;   // [lo, hi)
};
Span span(const void* p, int64_t elems, int64_t elem_bytes) {
    return Span{(uintptr_t)p, (uintptr_t)p + (uintptr_t)(elems * elem_bytes)};
}
bool overlap(Span a, Span b) { return a.lo < b.hi && b.lo < a.hi; }

// Shape checks shared by the three calls. Returns CGQA_OK, or sets *empty for B or T = 0.
int check_shape(int B, int T, int Hq, int Hkv, int d, float scale, bool* empty) {
    *empty = false;
    if (B < 0 || T < 0 || Hq < 1 || Hkv < 1) return CGQA_EINVAL;
    if (Hq % Hkv != 0) return CGQA_EINVAL;
    if (!(scale > 0.0f) || !isfinite(scale)) return CGQA_EINVAL;
    if (d != 64 && d != 128) return CGQA_EUNSUPPORTED;
    // Every element count must stay below 2^31 (kernel grids and row indices are int).
    const int64_t n_q = (int64_t)B * T * Hq * d;
    if (n_q >= ((int64_t)1 << 31)) return CGQA_EINVAL;
    if (B == 0 || T == 0) *empty = true;
    return CGQA_OK;
}

int finish(hipError_t e) {
    if (e != hipSuccess) {
        g_last_hip_error = (int)e;
        return CGQA_EHIP;
    }
    return CGQA_OK;
}

}  // namespace

extern "C" {

int attn_fwd(const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* o, float* lse,
             int B, int T, int Hq, int Hkv, int d, float scale, void* stream) {
    bool empty = false;
    int rc = check_shape(B, T, Hq, Hkv, d, scale, &empty);
    if (rc != CGQA_OK || empty) return rc;
    if (!q || !k || !v || !o || !lse) return CGQA_EINVAL;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse))
        return CGQA_EUNSUPPORTED;
    const int64_t nq = (int64_t)B * T * Hq * d, nkv = (int64_t)B * T * Hkv * d, nr = (int64_t)B * Hq * T;
    const Span so = span(o, nq, 2), sl = span(lse, nr, 4);
    const Span ins[3] = {span(q, nq, 2), span(k, nkv, 2), span(v, nkv, 2)};
    if (overlap(so, sl)) return CGQA_EINVAL;
    for (const Span& s : ins)
        if (overlap(s, so) || overlap(s, sl)) return CGQA_EINVAL;

    cgqa::FwdArgs a{};
    a.q = q; a.k = k; a.v = v; a.o = o; a.lse = lse;
    a.B = B; a.T = T; a.Hq = Hq; a.Hkv = Hkv; a.d = d;
    a.scale_log2 = (float)((double)scale * 1.4426950408889634);
    return finish(cgqa::launch_fwd(a, (hipStream_t)stream));
}

static int bwd_common(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* o,
                      const uint16_t* dO, const float* lse, const float* delta_in, float* delta_out,
                      float* dq, float* dk, float* dv, int B, int T, int Hq, int Hkv, int d, float scale,
                      void* stream, bool is_dq) {
    bool empty = false;
    int rc = check_shape(B, T, Hq, Hkv, d, scale, &empty);
    if (rc != CGQA_OK || empty) return rc;
    const int64_t nq = (int64_t)B * T * Hq * d, nkv = (int64_t)B * T * Hkv * d, nr = (int64_t)B * Hq * T;
    if (is_dq) {
        if (!q || !k || !v || !o || !dO || !lse || !delta_out || !dq) return CGQA_EINVAL;
        if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(dO) ||
            !aligned16(lse) || !aligned16(delta_out) || !aligned16(dq))
            return CGQA_EUNSUPPORTED;
        const Span outs[2] = {span(delta_out, nr, 4), span(dq, nq, 4)};
        const Span ins[6] = {span(q, nq, 2), span(k, nkv, 2), span(v, nkv, 2),
                             span(o, nq, 2), span(dO, nq, 2), span(lse, nr, 4)};
        if (overlap(outs[0], outs[1])) return CGQA_EINVAL;
        for (const Span& s : ins)
            if (overlap(s, outs[0]) || overlap(s, outs[1])) return CGQA_EINVAL;
    } else {
        if (!q || !k || !v || !dO || !lse || !delta_in || !dk || !dv) return CGQA_EINVAL;
        if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(dO) || !aligned16(lse) ||
            !aligned16(delta_in) || !aligned16(dk) || !aligned16(dv))
            return CGQA_EUNSUPPORTED;
        const Span outs[2] = {span(dk, nkv, 4), span(dv, nkv, 4)};
        const Span ins[6] = {span(q, nq, 2), span(k, nkv, 2), span(v, nkv, 2),
                             span(dO, nq, 2), span(lse, nr, 4), span(delta_in, nr, 4)};
        if (overlap(outs[0], outs[1])) return CGQA_EINVAL;
        for (const Span& s : ins)
            if (overlap(s, outs[0]) || overlap(s, outs[1])) return CGQA_EINVAL;
    }
    cgqa::BwdArgs a{};
    a.q = q; a.k = k; a.v = v; a.o = o; a.dO = dO; a.lse = lse;
    a.delta = is_dq ? delta_out : const_cast<float*>(delta_in);
    a.dq = dq; a.dk = dk; a.dv = dv;
    a.B = B; a.T = T; a.Hq = Hq; a.Hkv = Hkv; a.d = d;
    a.scale = scale;
    a.scale_log2 = (float)((double)scale * 1.4426950408889634);
    return finish(is_dq ? cgqa::launch_bwd_dq(a, (hipStream_t)stream)
                        : cgqa::launch_bwd_dkv(a, (hipStream_t)stream));
}

int attn_bwd_dq(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* o,
                const uint16_t* dO, const float* lse, float* delta, float* dq,
                int B, int T, int Hq, int Hkv, int d, float scale, void* stream) {
    return bwd_common(q, k, v, o, dO, lse, nullptr, delta, dq, nullptr, nullptr, B, T, Hq, Hkv, d,
                      scale, stream, true);
}

int attn_bwd_dkv(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* dO,
                 const float* lse, const float* delta, float* dk, float* dv,
                 int B, int T, int Hq, int Hkv, int d, float scale, void* stream) {
    return bwd_common(q, k, v, nullptr, dO, lse, delta, nullptr, nullptr, dk, dv, B, T, Hq, Hkv, d,
                      scale, stream, false);
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
