// Host-side launch interface between the C-ABI entry points and the kernels.
// Arguments arrive here already validated (shapes, alignment, d in {64, 128}).
//
// Tensor layout: element (b, t, h, c) of a [B, T, H, d] tensor with row stride rs (elements
// between consecutive tokens, rs >= H*d) sits at (b*T + t)*rs + h*d + c; rs = H*d is the
// contiguous layout. LSE and delta are always [B, Hq, T].
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

namespace cgqa {

// Floor division by a divisor fixed at launch, on the scalar unit. For 0 <= n < 2^31 and
// 1 <= d < 2^31, q0 = floor(n m / 2^32) with m = floor((2^32 - 1) / d) is floor(n / d) or
// one less (n m / 2^32 lies in (n/d - 1, n/d]), and one comparison fixes it. The
// compiler's general 32-bit division runs on the vector ALU (a float reciprocal, fix-ups and
// readfirstlane) even for wave-uniform operands; this one stays in scalar registers.
struct UDiv {
    unsigned m;
    int d;
};
inline UDiv make_udiv(int d) { return {0xFFFFFFFFu / (unsigned)d, d}; }
__device__ __forceinline__ int udiv(int n, const UDiv& v) {
    unsigned q = __umulhi((unsigned)n, v.m);
    if ((unsigned)n - q * (unsigned)v.d >= (unsigned)v.d) ++q;
    return (int)q;
}
// The divisors of the kernels' workgroup maps (set by the C-ABI layer before every launch):
// G = Hq / Hkv; per-tile workgroups of one XCD ((B Hkv / 8) G when slices are grouped on
// XCDs); B Hq; B Hkv.
struct MapDivs {
    int G;
    UDiv g, hkv, hq, tile, bhq, bhkv;
};
inline MapDivs make_map_divs(int B, int Hq, int Hkv) {
    const int G = Hq / Hkv;
    const int tile = ((B * Hkv) >> 3) * G;
    return {G, make_udiv(G), make_udiv(Hkv), make_udiv(Hq), make_udiv(tile > 0 ? tile : 1),
            make_udiv(B * Hq), make_udiv(B * Hkv)};
}

struct FwdArgs {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    uint16_t* o;
    float* lse;
    int B, T, Hq, Hkv, d;
    int q_rs, kv_rs, o_rs;   // row strides of Q, of K and V, of O (elements)
    float scale_log2;   // scale * log2(e): scores in log2 units
    int n_qtiles;       // set by the launcher: query tiles per (batch, head)
    int n_pairs;        // set by the launcher: B * Hkv (batch, kv head) slices
    int xcd_group;      // set by the launcher: keep each slice's tiles on one XCD
    const float* rope_cos;   // rotary tables [T][d/2] when the kernel turns Q and K itself
    const float* rope_sin;   // (attn_fwd_rope); unused otherwise
    MapDivs div;        // set by the C-ABI layer
    // Set by the launcher: when perm_n > 0, workgroup x of XCD x % 8 takes the tile at
    // position perm[x >> 3] of the heaviest-first order instead of position x >> 3 (see
    // balance_one_round).
    int perm_n;
    unsigned char perm[256];
};

struct BwdArgs {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    const uint16_t* o;
    const uint16_t* dO;
    const float* lse;
    float* delta;       // written by the dq kernel, read by the dkv kernel
    float* do_absmax;   // [B][Hq][ceil(T/32)]: largest |dO| per 32-row block (dq writes, dkv reads)
    void* dq;           // fp32, or bf16 when grad_bf16
    void* dk;
    void* dv;
    int B, T, Hq, Hkv, d;
    int q_rs, kv_rs, o_rs, do_rs;   // input row strides (elements)
    int dq_rs, dkv_rs;              // output row strides (elements of the output type)
    int grad_bf16;                  // 1: dQ, dK, dV rounded to bf16 (nearest even)
    const float* rope_cos;          // rotary tables [T][d/2]: dQ and dK are turned back to
    const float* rope_sin;          // the unrotated inputs' frame (null: no rotation)
    float scale;        // softmax scale (dS carries it into dQ and dK)
    float scale_log2;   // scale * log2(e)
    int n_tiles;        // set by the launcher
    int zigzag;         // dK/dV: deal key blocks in zig-zag order (set by the launcher)
    int xcd_group;      // dQ: keep each (batch, kv head) slice on one XCD (set by the launcher)
    MapDivs div;        // set by the C-ABI layer
};

// Naive attention (attn_naive.hip): contiguous tensors, fp32 workspace p of B*Hq*T*T
// floats, 1 <= d <= 128.
struct NaiveArgs {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    const uint16_t* dO;   // backward only
    uint16_t* o;          // forward only
    float* lse;           // forward only (null in the backward, which recomputes P)
    float* delta;         // backward only
    float* dq;
    float* dk;
    float* dv;
    float* p;             // workspace
    int B, T, Hq, Hkv, d;
    float scale;
};

// Matrix product C = A B^T (+ R) with layout flags (gemm.hip). K % 32 == 0; A_KM needs
// M % 8 == 0, B_KN needs N % 8 == 0; M*K, N*K, M*N < 2^31.
struct GemmArgs {
    const uint16_t* a;    // [M][K], or [K][M] when a_km
    const uint16_t* b;    // [N][K], or [K][N] when b_kn
    void* c;              // [M][N] fp32, or bf16 when c_bf16
    const float* r;       // [M][N] fp32 added to the product, or null; may be c
    int M, N, K;
    int a_km, b_kn, c_bf16;
    float* ws;            // workspace for a K split, or null (no split)
    size_t ws_bytes;
    int tiles_m, tiles_n; // set by the launcher
    int ksplit, kps;      // set by the launcher: splits of K and 32-k tiles per split
};
// Splits of K the launcher uses for this shape and workspace size (1: none).
int gemm_splits(int M, int N, int K, size_t ws_bytes);
// Matrix-core calibration (calib.hip): `blocks` workgroups of kCalibThreads threads; each
// thread stores iters / 64 to sink[block * kCalibThreads + thread]; clocks (or null) gets
// block 0's loop time in shader clocks and in 100 MHz ticks.
constexpr int kCalibThreads = 256;
hipError_t launch_calib_mfma(float* sink, unsigned long long* clocks, int blocks, int iters, hipStream_t stream);
double calib_mfma_flops(int blocks, int iters);
// Bytes of the static split-K scratch of the allocation-free GEMM (per device), and its
// device address on the current device (looked up once per device).
constexpr size_t kGemmScratchBytes = (size_t)16 << 20;
hipError_t gemm_scratch(float** ptr);
// Floats per split's partial product in the workspace: M*N rounded up to a multiple of 4.
__host__ __device__ inline size_t gemm_slice_floats(int M, int N) { return ((size_t)M * N + 3) & ~(size_t)3; }

// Rotary embedding of Q and K (rope.hip): out = R(t) in per pair, bf16.
struct RopeArgs {
    const uint16_t* q;
    const uint16_t* k;
    uint16_t* q_out;      // may be q itself (same stride)
    uint16_t* k_out;      // may be k itself
    const float* cos;     // [T][d/2]
    const float* sin;
    int B, T, Hq, Hkv, d;
    int q_rs, k_rs, qo_rs, ko_rs;   // row strides (elements)
};
hipError_t launch_rope(const RopeArgs& a, hipStream_t stream);

hipError_t launch_fwd(const FwdArgs& a, hipStream_t stream);
// The forward with the rotary embedding applied to Q and K as they are loaded.
hipError_t launch_fwd_rope(const FwdArgs& a, hipStream_t stream);
// Forward with every query block's keys split over two waves (attn_fwd_par.hip), for
// d = 64 grids that would not fill the chip with the tiled kernel.
bool fwd_split_keys_chosen(const FwdArgs& a);
hipError_t launch_fwd_split_keys(const FwdArgs& a, hipStream_t stream);
hipError_t launch_bwd_dq(const BwdArgs& a, hipStream_t stream);
hipError_t launch_bwd_dkv(const BwdArgs& a, hipStream_t stream);
hipError_t launch_naive_fwd(const NaiveArgs& a, hipStream_t stream);
hipError_t launch_naive_bwd(const NaiveArgs& a, hipStream_t stream);
hipError_t launch_gemm(const GemmArgs& a, hipStream_t stream);

// CUs per XCD of the current device (gfx950: eight XCDs); 0 if the runtime cannot say.
inline int cus_per_xcd() {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return 0;
    return n / 8;
}

// Dispatch order of a grid that fits the chip in one residency round (every workgroup
// resident from the start). On gfx950 the workgroups of one XCD go to its C CUs in launch
// order, one per CU per pass: the workgroups with local index i, C + i, 2C + i, ... of an
// XCD share one CU (measured: a probe that recorded the hardware ids of every wave of such
// a launch). With tiles launched heaviest first, the CU that receives the heaviest tile of
// the first pass also receives the heaviest of every later pass, and the kernel lasts as
// long as that CU's sum. Here the passes are filled greedily instead: pass by pass, the
// heaviest remaining tiles go to the CUs with the least work so far. weight(p), p in
// [0, L), is the work of position p of the heaviest-first order and must not increase with
// p. Writes perm[local] = position and returns L, or returns 0 (keep the heaviest-first
// order) when the grid is larger than one round or than the table. Any permutation gives
// the same results; only the balance changes. No allocation: fixed arrays on the stack.
template <typename W>
inline int balance_one_round(unsigned char* perm, int L, int C, int S, W weight) {
    constexpr int kMax = 256;
    if (L <= 0 || C <= 0 || C > kMax || L > C * S || L > kMax) return 0;
    const int passes = (L + C - 1) / C;
    long load[kMax] = {};
    int cu_of[kMax], order[kMax], label[kMax];
    for (int r = 0; r < passes; ++r) {
        for (int c = 0; c < C; ++c) order[c] = c;
        std::stable_sort(order, order + C, [&](int a, int b) { return load[a] < load[b]; });
        const int p0 = r * C, n = std::min(C, L - p0);
        for (int k = 0; k < n; ++k) {
            cu_of[p0 + k] = order[k];
            load[order[k]] += weight(p0 + k);
        }
    }
    // The CUs that take a tile in a last, partial pass must be those that local indices
    // r*C + 0 .. r*C + n-1 reach: relabel them 0 .. n-1 (the same labels in every pass).
    for (int c = 0; c < C; ++c) label[c] = -1;
    const int last0 = (passes - 1) * C, nlast = L - last0;
    int next = 0;
    for (int k = 0; k < nlast; ++k) label[cu_of[last0 + k]] = next++;
    for (int c = 0; c < C; ++c)
        if (label[c] < 0) label[c] = next++;
    for (int p = 0; p < L; ++p) perm[(p / C) * C + label[cu_of[p]]] = (unsigned char)p;
    return L;
}

}  // namespace cgqa
