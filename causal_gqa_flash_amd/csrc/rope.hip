// Rotary position embedding of queries and keys (page "A transformer in PTX", section
// "The model": queries and keys are rotated with RoPE, in place in the bf16 QKV buffer,
// between the fused QKV matmul and attention). Pair i = (x[2i], x[2i+1]) of every head
// of token t turns by the angle with cosine cos[t][i] and sine sin[t][i]:
//   y[2i] = x[2i] cos - x[2i+1] sin,   y[2i+1] = x[2i] sin + x[2i+1] cos,
// stored as bf16, rounded once from the exact value (to nearest, ties to even).
//
// Exact rounding: see rope_turn8 (the forward with the rotation in its tile loads uses the
// same arithmetic, so both give the same bits).
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
        const f32x4 cs = *reinterpret_cast<const f32x4*>(a.cos + (size_t)t * half + dim / 2);
        const f32x4 sn = *reinterpret_cast<const f32x4*>(a.sin + (size_t)t * half + dim / 2);
        const u32x4 out = rope_turn8(raw, cs, sn);
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
