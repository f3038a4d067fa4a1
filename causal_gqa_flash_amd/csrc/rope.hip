// Rotary position embedding of queries and keys (page "A transformer in PTX", section
// "The model": queries and keys are rotated with RoPE, in place in the bf16 QKV buffer,
// between the fused QKV matmul and attention). Pair i = (x[2i], x[2i+1]) of every head
// of token t turns by the angle with cosine cos[t][i] and sine sin[t][i]:
//   y[2i] = x[2i] cos - x[2i+1] sin,   y[2i+1] = x[2i] sin + x[2i+1] cos,
// stored as bf16, rounded once from the exact value (to nearest, ties to even).
//
// Exact rounding: a bf16 input times an fp32 table value has at most 32 significant bits,
// so it is exact in fp64, and fma(x0, c, -(x1 s)) in fp64 rounds the exact y a single time,
// to 53 bits. Rounding that to fp32 and then to bf16 can only go wrong where the fp32
// value lands exactly on a bf16 tie (the low 16 bits 0x8000); there the fp64 value says
// on which side of the tie y lies, and the fp32 value is nudged one unit that way before
// its rounding to bf16. The one case left is an exact y within 2^-53 of a tie without
// being one (bits 10 to 53 of its significand all equal), which fp64 cannot resolve.
//
// A memory-bound pass: each thread turns 8 consecutive elements (4 pairs, one 16-byte
// load and store) with 4 cosines and 4 sines (16-byte loads of the tables, which stay in
// L2). Output may be the input itself (each thread reads its elements before writing
// them), so the pass can run in place on a packed QKV buffer.
#include "cgqa_device.hpp"
#include "cgqa_launch.hpp"

namespace cgqa {
namespace {

constexpr int kThreads = 256;

// An fp32 value whose rounding to bf16 (nearest even) is that of the fp64 y: y rounded
// to fp32, moved one unit toward y when it sits exactly on a bf16 rounding tie.
__device__ __forceinline__ float to_bf16_exact(double y) {
    const float f = (float)y;
    unsigned u = __float_as_uint(f);
    if ((u & 0xFFFFu) == 0x8000u) {
        const double fd = (double)f;
        if (y != fd) u = ((y > fd) == (f > 0.0f)) ? u + 1u : u - 1u;
    }
    return __uint_as_float(u);
}

__global__ __launch_bounds__(kThreads) void rope_qk_kernel(RopeArgs a) {
    // 8-element chunks per token; B*T*(Hq+Hkv)*d < 2^31, so 32-bit index arithmetic.
    const unsigned cq = (unsigned)(a.Hq * a.d / 8), cpr = cq + (unsigned)(a.Hkv * a.d / 8);
    const unsigned total = (unsigned)a.B * (unsigned)a.T * cpr;
    const int half = a.d / 2;
    for (unsigned c = blockIdx.x * kThreads + threadIdx.x; c < total; c += gridDim.x * kThreads) {
        const unsigned row = c / cpr;      // b * T + t
        const unsigned j = c - row * cpr;
        const int t = (int)(row % (unsigned)a.T);
        const bool isq = j < cq;
        const int e = 8 * (int)(isq ? j : j - cq);            // element within the token's heads
        const uint16_t* src = isq ? a.q + (size_t)row * a.q_rs + e : a.k + (size_t)row * a.k_rs + e;
        uint16_t* dst = isq ? a.q_out + (size_t)row * a.qo_rs + e : a.k_out + (size_t)row * a.ko_rs + e;
        const int dim = e % a.d;
        const u32x4 raw = load16(src);
        const bf16x8 x = __builtin_bit_cast(bf16x8, raw);
        const f32x4 cs = *reinterpret_cast<const f32x4*>(a.cos + (size_t)t * half + dim / 2);
        const f32x4 sn = *reinterpret_cast<const f32x4*>(a.sin + (size_t)t * half + dim / 2);
        f32x4 lo, hi;
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const double x0 = (double)(float)x[2 * p], x1 = (double)(float)x[2 * p + 1];
            const double c = (double)cs[p], sn_p = (double)sn[p];
            const double y0 = fma(x0, c, -(x1 * sn_p));
            const double y1 = fma(x0, sn_p, x1 * c);
            if (p < 2) { lo[2 * p] = to_bf16_exact(y0); lo[2 * p + 1] = to_bf16_exact(y1); }
            else { hi[2 * p - 4] = to_bf16_exact(y0); hi[2 * p - 3] = to_bf16_exact(y1); }
        }
        const bf16x4 blo = __builtin_convertvector(lo, bf16x4), bhi = __builtin_convertvector(hi, bf16x4);
        u32x4 out;
        const u32x2 wlo = __builtin_bit_cast(u32x2, blo), whi = __builtin_bit_cast(u32x2, bhi);
        out[0] = wlo[0]; out[1] = wlo[1]; out[2] = whi[0]; out[3] = whi[1];
        *reinterpret_cast<u32x4*>(dst) = out;
    }
}

}  // namespace

hipError_t launch_rope(const RopeArgs& a, hipStream_t stream) {
    const long total = (long)a.B * a.T * (a.Hq + a.Hkv) * (a.d / 8);
    const long blocks = (total + kThreads - 1) / kThreads;
    const unsigned grid = (unsigned)(blocks < 16384 ? (blocks > 0 ? blocks : 1) : 16384);
    hipLaunchKernelGGL(rope_qk_kernel, dim3(grid), dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace cgqa
