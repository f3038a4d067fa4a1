// Backward kernels of causal grouped-query flash attention for gfx950.
//
// Method (page "A transformer in PTX", sections "Flash attention" and "The same bits
// every time"): the backward is two kernels. Both recompute the probabilities from the
// scores and the saved log-sum-exp instead of storing them. The dQ kernel owns a block
// of queries; the dK/dV kernel owns a block of keys and loops over all query heads
// that share its key/value head. No float atomics: every output element has one
// writer that adds its terms in a fixed order, so two runs give the same bits.
//
// For the loss L = sum(O * dO):
//   P = exp(S - LSE), dP = dO V^T, D_i = sum_j P_ij dP_ij (= dO_i . O_i),
//   dS = P * (dP - D), dQ = scale * dS K, dK = scale * dS^T Q, dV = P^T dO.
// In log2 units P = 2^(S * scale * log2(e) - LSE * log2(e)).
//
// Precision. The products that take P or dS run on the fp16 matrix core with fp32
// accumulation: their other operands are converted from bf16 to fp16 (exact for
// magnitudes in [2^-14, 65504]), and P and dS are rounded to fp16, which carries three
// more bits than bf16. dS and dO scale with the loss: gradients into attention are often
// far below fp16's normal range (2^-14). So they are scaled by exact powers of two before
// the rounding and the products are scaled back in fp32 at the end: in the dQ kernel each
// query row by the inverse of its own largest |dO| (dQ row i only sums row i's terms); in
// the dK/dV kernel, whose sums run over many query rows, every row of a (batch, kv head)
// group by one scale, the one that brings the group's largest |dO| into [1, 2). The dQ
// kernel, which reads every dO row anyway, publishes the largest |dO| of each block of
// 32 rows; the dK/dV kernel reduces its group's blocks before its loop. Scaled dO then
// stays below 2 and dS below 65504 as long as every row of V has sum_c |V_c| < 16000.
// Power-of-two scaling commutes with rounding in the normal range, so a power-of-two
// factor on dO moves every gradient by exactly that factor.
// D has to be accurate to the fp32 level: the one the bf16 output O gives (D~ = dO . O_bf16) is off by the rounding of O, and that error
// is multiplied by K in dQ and by Q in dK. The dQ kernel therefore forms dS~ with D~
// (known before its loop), accumulates the exact D = sum_j P_ij dP_ij on the side and
// K_bar = sum_j P_ij K_j with one more product, and finishes with
//   dQ = scale * (dS~ K - (D - D~) K_bar),
// which is the same sum. It writes that exact D to `delta` for the dK/dV kernel.
//
// gfx950 layout choices:
//  * dQ kernel: like the forward, scores are computed transposed (S^T = K Q^T, dP^T =
//    V dO^T) so each lane owns one query; dS^T and P^T then feed dQ^T += K^T dS^T and
//    K_bar^T += K^T P^T straight from the accumulator registers, with K^T read from
//    the row-major K tile by the transposing LDS read.
//  * dK/dV kernel: scores are computed untransposed (S = Q K^T, dP = dO V^T) so each
//    lane owns one key; P and dS feed dV^T += dO^T P and dK^T += Q^T dS from the
//    accumulator registers, with dO^T and Q^T read transposed from the staged tiles.
//    K and V of the lane's key stay in registers for the whole loop.
#include "cgqa_device.hpp"
#include "cgqa_launch.hpp"

namespace cgqa {

// ------------------------------------------------------------------------ dQ kernel
template <int D, int NQB, int BN, int NW>
struct DqCfg {
    static constexpr int kThreads = NW * 64;
    static constexpr int kBM = NW * 32 * NQB;
    static constexpr int kKD = D / 16;
    static constexpr int kNKB = BN / 32;
    static constexpr int kMB = D / 32;
    static constexpr int kPitch = D * 2 + 16;     // K (fp16) and V (bf16) rows in LDS
    static constexpr int kTile = BN * kPitch;
    static constexpr int kStage = 2 * kTile;
    static constexpr int kLds = 2 * kStage;
    static constexpr int kChunks = BN * D / 8;
    static constexpr int kPerThread = kChunks / kThreads;
    static_assert(D == 64 || D == 128, "head dim");
    static_assert(kChunks % kThreads == 0, "tile load must split evenly over the threads");
    static_assert(kLds <= 160 * 1024, "LDS budget");
};

// Query tile and (batch, head) of dQ workgroup bid, heaviest query tiles first. Workgroup
// x runs on XCD x mod 8; when the (batch, kv head) slices split evenly over the eight XCDs,
// every head and tile of a slice goes to the slice's XCD, whose L2 then serves its K and V
// to all heads of the group (otherwise the group's heads land on different XCDs and each
// fetches the slice's K and V from HBM).
struct DqTile { int qt, b, h; };
__device__ inline DqTile dq_tile(const BwdArgs& a, int bid) {
    const int G = a.div.G;
    if (a.xcd_group) {
        const int xcd = bid & 7;
        const int per_qt = a.div.tile.d;                 // workgroups per query tile on one XCD
        const int local = bid >> 3;
        const int jt = udiv(local, a.div.tile);
        const int rem = local - jt * per_qt;
        const int sl = udiv(rem, a.div.g);
        const int p = xcd + 8 * sl;                      // slice b * Hkv + g
        const int b = udiv(p, a.div.hkv);
        return {a.n_tiles - 1 - jt, b, (p - b * a.Hkv) * G + (rem - sl * G)};
    }
    const int jt = udiv(bid, a.div.bhq);
    const int bh = bid - jt * (a.B * a.Hq);
    const int b = udiv(bh, a.div.hq);
    return {a.n_tiles - 1 - jt, b, bh - b * a.Hq};
}

template <int D, int NQB, int BN, int NW>
__global__ __launch_bounds__(NW * 64) void attn_bwd_dq_kernel(BwdArgs a_in) {
    BwdArgs a = a_in;
    pin_args(a);   // all argument loads at entry (see pin_args)
    using C = DqCfg<D, NQB, BN, NW>;
    __shared__ __attribute__((aligned(16))) char smem[C::kLds];

    const int T = a.T, Hq = a.Hq;
    const DqTile wg = dq_tile(a, blockIdx.x);
    const int qt = wg.qt, b = wg.b, h = wg.h;
    const int g = udiv(h, a.div.g);

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int n = lane & 31, hl = lane >> 5;
    const int q0 = qt * C::kBM;
    const int qw = q0 + wave * 32 * NQB;

    const size_t kv_stride = (size_t)a.kv_rs;
    const uint16_t* qrow0 = a.q + (size_t)b * T * a.q_rs + (size_t)h * D;
    const uint16_t* dorow0 = a.dO + (size_t)b * T * a.do_rs + (size_t)h * D;
    const uint16_t* orow0 = a.o + (size_t)b * T * a.o_rs + (size_t)h * D;
    const uint16_t* kbase = a.k + (size_t)b * T * a.kv_rs + (size_t)g * D;
    const uint16_t* vbase = a.v + (size_t)b * T * a.kv_rs + (size_t)g * D;

    // Q (fp16) and dO (bf16, as given) as B operands (lane: query n, dims 16*kd + 8*hl
    // .. +7), D~ and LSE. dP = V dO^T multiplies inputs only, so it runs in bf16
    // exactly as in fp16; the products with computed P and dS~ use K in fp16.
    f16x8 qreg[NQB][C::kKD];
    bf16x8 doreg[NQB][C::kKD];
    float dtilde[NQB], lse2[NQB], dexact[NQB], dsc[NQB], dsc_inv[NQB], dts[NQB];
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
        const int row = qw + 32 * qb + n;
        float part = 0.0f;
        unsigned dmax = 0;
#pragma unroll
        for (int kd = 0; kd < C::kKD; ++kd) {
            u32x4 xq = {0u, 0u, 0u, 0u}, xd = {0u, 0u, 0u, 0u}, xo = {0u, 0u, 0u, 0u};
            if (row < T) {
                const int col = 16 * kd + 8 * hl;
                xq = load16(qrow0 + (size_t)row * a.q_rs + col);
                xd = load16(dorow0 + (size_t)row * a.do_rs + col);
                xo = load16(orow0 + (size_t)row * a.o_rs + col);
            }
            qreg[qb][kd] = bf16x8_to_f16(xq);
            doreg[qb][kd] = __builtin_bit_cast(bf16x8, xd);
            dmax = max(dmax, bf16x8_absmax_bits(xd));
            const bf16x8 dv8 = __builtin_bit_cast(bf16x8, xd);
            const bf16x8 ov8 = __builtin_bit_cast(bf16x8, xo);
#pragma unroll
            for (int s = 0; s < 8; ++s) part += (float)dv8[s] * (float)ov8[s];
        }
        part += swap_halves(part);
        dtilde[qb] = part;
        // dS of this row is scaled by 2^k (largest |dO| of the row into [1, 2)) before its
        // fp16 rounding, and dQ~ scaled back at the store.
        dmax = max(dmax, (unsigned)__shfl_xor((int)dmax, 32, 64));
        // The block's largest |dO| (its 32 rows), published for the dK/dV pass.
        const unsigned bmax = wave_max_u32(dmax);
        if (lane == 0 && qw + 32 * qb < T)
            a.do_absmax[((size_t)b * Hq + h) * ((T + 31) / 32) + (qw + 32 * qb) / 32] = __uint_as_float(bmax << 16);
        const Pow2Scale ps = pow2_normalizer(dmax);
        dsc[qb] = ps.s;
        dsc_inv[qb] = ps.inv;
        dts[qb] = part * ps.s;
        dexact[qb] = 0.0f;
        lse2[qb] = row < T ? a.lse[((size_t)b * Hq + h) * T + row] * kLog2e : 0.0f;
    }

    f32x16 dqacc[NQB][C::kMB], kbar[NQB][C::kMB];
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
        for (int mb = 0; mb < C::kMB; ++mb) { dqacc[qb][mb] = zero16(); kbar[qb][mb] = zero16(); }

    const int kv_end = min(T, q0 + C::kBM);
    const int ntiles = (kv_end + BN - 1) / BN;

    u32x4 kst[C::kPerThread], vst[C::kPerThread];
    auto load_tile = [&](int j0) {
#pragma unroll
        for (int i = 0; i < C::kPerThread; ++i) {
            const int c = tid + i * C::kThreads;
            const int row = c / (D / 8), col = c % (D / 8);
            const int key = j0 + row;
            u32x4 xk = {0u, 0u, 0u, 0u}, xv = {0u, 0u, 0u, 0u};
            if (key < T) {
                xk = load16(kbase + (size_t)key * kv_stride + col * 8);
                xv = load16(vbase + (size_t)key * kv_stride + col * 8);
            }
            kst[i] = xk;
            vst[i] = xv;
        }
    };
    auto store_tile = [&](int buf) {
        char* ks = smem + buf * C::kStage;
        char* vs = ks + C::kTile;
#pragma unroll
        for (int i = 0; i < C::kPerThread; ++i) {
            const int c = tid + i * C::kThreads;
            const int row = c / (D / 8), col = c % (D / 8);
            store16(ks + row * C::kPitch + col * 16, bf16x8_to_f16_bits(kst[i]));
            store16(vs + row * C::kPitch + col * 16, vst[i]);
        }
    };

    load_tile(0);
    store_tile(0);
    __syncthreads();

    const int tr_row = (lane & 15) >> 2;
    const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);

    // One key tile against this wave's queries, from LDS buffer U. Only tiles that
    // reach past the wave's first query need the causal mask (MASK).
    auto tile = [&](auto Uc, auto Mc, int j0) {
        constexpr int U = decltype(Uc)::value;
        constexpr bool MASK = decltype(Mc)::value;
        const char* ks = smem + U * C::kStage;
        const char* vs = ks + C::kTile;
        f32x16 s[C::kNKB][NQB], dp[C::kNKB][NQB];
#pragma unroll
        for (int kb = 0; kb < C::kNKB; ++kb) {
#pragma unroll
            for (int qb = 0; qb < NQB; ++qb) { s[kb][qb] = zero16(); dp[kb][qb] = zero16(); }
#pragma unroll
            for (int kd = 0; kd < C::kKD; ++kd) {
                const int off = (32 * kb + n) * C::kPitch + (16 * kd + 8 * hl) * 2;
                const f16x8 ka = lds_read8_f16(ks + off);
                const bf16x8 va = lds_read8(vs + off);
#pragma unroll
                for (int qb = 0; qb < NQB; ++qb) {
                    s[kb][qb] = mfma32x32x16(ka, qreg[qb][kd], s[kb][qb]);
                    dp[kb][qb] = mfma32x32x16(va, doreg[qb][kd], dp[kb][qb]);
                }
            }
        }
        // P^T into s, dS~^T into dp; the exact D on the side.
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb) {
            const int rel = j0 + 4 * hl - (qw + 32 * qb + n);   // key - query at kb = i = 0
#pragma unroll
            for (int kb = 0; kb < C::kNKB; ++kb) {
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    float p = exp2_fast(fmaf(s[kb][qb][i], a.scale_log2, -lse2[qb]));
                    if constexpr (MASK) {
                        if (rel + 32 * kb + 8 * (i >> 2) + (i & 3) > 0) p = 0.0f;
                    }
                    dexact[qb] = fmaf(p, dp[kb][qb][i], dexact[qb]);
                    dp[kb][qb][i] = p * fmaf(dp[kb][qb][i], dsc[qb], -dts[qb]);
                    s[kb][qb][i] = p;
                }
            }
        }
        // dQ~^T += K^T dS~^T and K_bar^T += K^T P^T (B from registers, A = K^T read
        // transposed from the K tile).
#pragma unroll
        for (int kb = 0; kb < C::kNKB; ++kb) {
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                f16x8 db[NQB], pb[NQB];
#pragma unroll
                for (int qb = 0; qb < NQB; ++qb) {
                    db[qb] = t == 0 ? pack_lo_f16(dp[kb][qb]) : pack_hi_f16(dp[kb][qb]);
                    pb[qb] = t == 0 ? pack_lo_f16(s[kb][qb]) : pack_hi_f16(s[kb][qb]);
                }
                const int r0 = 32 * kb + 16 * t + 4 * hl + tr_row;
#pragma unroll
                for (int mb = 0; mb < C::kMB; ++mb) {
                    const char* p0 = ks + r0 * C::kPitch + (32 * mb + tr_col) * 2;
                    const f16x8 kt = concat(lds_read_tr4_f16(p0), lds_read_tr4_f16(p0 + 8 * C::kPitch));
#pragma unroll
                    for (int qb = 0; qb < NQB; ++qb) {
                        dqacc[qb][mb] = mfma32x32x16(kt, db[qb], dqacc[qb][mb]);
                        kbar[qb][mb] = mfma32x32x16(kt, pb[qb], kbar[qb][mb]);
                    }
                }
            }
        }
    };

    // Two LDS buffers; the loop is unrolled by two so each buffer's offsets are
    // immediates. The next tile's global loads run during the current tile.
    for (int jt0 = 0; jt0 < ntiles; jt0 += 2) {
        static_for<2>([&](auto Uc) {
            constexpr int U = decltype(Uc)::value;
            const int jt = jt0 + U;
            if (jt >= ntiles) return;
            const int j0 = jt * BN;
            if (jt + 1 < ntiles) load_tile(j0 + BN);
            if (qw + 32 * NQB - 1 >= j0) {
                if (j0 + BN - 1 > qw) tile(Uc, std::true_type{}, j0);
                else tile(Uc, std::false_type{}, j0);
            }
            if (jt + 1 < ntiles) store_tile(1 - U);
            lds_barrier();
        });
    }

#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
        const int query = qw + 32 * qb + n;
        const float dfull = dexact[qb] + swap_halves(dexact[qb]);
        if (query >= T) continue;
        if (hl == 0) a.delta[((size_t)b * Hq + h) * T + query] = dfull;
        const float corr = dfull - dtilde[qb];
        const size_t drow = ((size_t)b * T + query) * a.dq_rs + (size_t)h * D;
        // Rotary tables of this row, all loaded before the first store.
        RopeCS rt[C::kMB][4];
        if (a.rope_cos) {
#pragma unroll
            for (int mb = 0; mb < C::kMB; ++mb)
#pragma unroll
                for (int u = 0; u < 4; ++u) rt[mb][u] = rope_load(a.rope_cos, a.rope_sin, query, D / 2, 32 * mb + 8 * u + 4 * hl);
        }
#pragma unroll
        for (int mb = 0; mb < C::kMB; ++mb)
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                f32x4 x;
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    x[r] = a.scale * fmaf(-corr, kbar[qb][mb][4 * u + r], dqacc[qb][mb][4 * u + r] * dsc_inv[qb]);
                if (a.rope_cos) x = rope_back4(x, rt[mb][u]);
                store_out4(a.dq, drow + 32 * mb + 8 * u + 4 * hl, x, a.grad_bf16);
            }
    }
}

// ---------------------------------------------------------------------- dK/dV kernel
// One workgroup owns NKW blocks of 32 keys of one key/value head. Its waves form HS
// head slots of NKW waves: slot s handles the query heads s, s + HS, ... of the group
// (ascending), each wave of a slot one key block, and the waves of a slot share staged
// Q/dO tiles of their current head. All slots step through the query tiles together,
// from the tile holding the workgroup's earliest key to the last. At the end the slots'
// partial dK and dV of each key are summed through LDS in ascending slot order: every
// output element still has one writer and a fixed summation order.
// Which key blocks a workgroup gets: the causal work of block kb falls with kb (it
// meets T - 32kb queries). When the grid is several rounds deep, consecutive blocks
// per workgroup with the early (heavy) ones launched first balance well. When it is a
// single round, the blocks are dealt in zig-zag order (0, last, 1, last-1, ...) so every
// workgroup gets early and late blocks and about the same work; a wave's block is then
// rotated by its slot so that the waves sharing a SIMD mix early and late blocks.
template <int D, int BQ, int NKW, int HS, int NR>
struct DkvCfg {
    static constexpr int kThreads = NKW * HS * 64;
    static constexpr int kKD = D / 16;
    static constexpr int kMB = D / 32;
    // Raw ring (NR stages, filled by DMA two steps ahead when NR = 3): Q and dO rows as
    // bf16, then lse and delta as fp32.
    static constexpr int kRawRow = D * 2;
    static constexpr int kRawTile = BQ * kRawRow;
    static constexpr int kRawStage = 2 * kRawTile + 2 * BQ * 4;
    // Converted double buffer: Q and dO rows as fp16 (padded pitch), lse * log2(e)
    // (+inf past T) and delta (0 past T).
    static constexpr int kPitch = D * 2 + 16;
    static constexpr int kTile = BQ * kPitch;
    static constexpr int kConvStage = 2 * kTile + 2 * BQ * 4;
    static constexpr int kSlot = NR * kRawStage + 2 * kConvStage;
    static constexpr int kSlotThreads = NKW * 64;
    static constexpr int kTileLoads = kRawTile / 1024 / NKW;     // per tensor, per wave
    static constexpr int kStatLanes = 2 * BQ / NKW;              // 4-byte DMA lanes per wave
    // A slot of one wave loads lse and delta itself: two 4-byte loads, each under half of
    // the lanes (a load's base is wave-uniform).
    static constexpr int kStatLoads = kStatLanes > BQ ? 2 : 1;
    static constexpr int kVmPerStep = 2 * kTileLoads + kStatLoads;   // DMA instructions per wave
    static constexpr int kConvChunks = kRawTile / 16 / kSlotThreads;   // per tensor, per thread
    // Reduction area: one 32-dim accumulator block (16 floats) per lane of every wave
    // of slots 1 .. HS-1; the blocks are reduced one after another.
    static constexpr int kRedBytes = NKW * (HS - 1) * 64 * 16 * 4;
    static constexpr int kLds = (HS * kSlot > kRedBytes) ? HS * kSlot : kRedBytes;
    static_assert(D == 64 || D == 128, "head dim");
    static_assert(BQ == 32, "one 32-query block per step");
    static_assert(NR == 2 || NR == 3, "raw ring depth");
    static_assert(kRawTile % (1024 * NKW) == 0, "tile DMA must split evenly over a slot");
    static_assert(kStatLanes >= 1 && kStatLanes <= 64 && (2 * BQ) % NKW == 0, "stat DMA lanes");
    static_assert(kRawTile % (16 * kSlotThreads) == 0, "conversion must split evenly");
    static_assert(kThreads <= 1024, "workgroup size");
    static_assert(kLds <= 160 * 1024, "LDS budget");
};

// SAME_QDO: Q and dO have the same row stride (every contiguous call), so their DMA
// shares one set of lane offsets and one cursor offset. BF16OUT: dK and dV are written
// as bf16. ROPE: dK is turned back by the rotary tables. (Compile-time choices: run-time
// ones cost this kernel registers it has not got.)
template <int D, int BQ, int NKW, int HS, int NR, bool SAME_QDO, bool BF16OUT, bool ROPE>
__global__ __launch_bounds__(NKW * HS * 64) void attn_bwd_dkv_kernel(BwdArgs a_in) {
    BwdArgs a = a_in;
    // d = 128: the arguments first used after the prologue are loaded at entry too (see
    // pin_args; 3% faster at B4 T4096 Hq32). At d = 64 the same change moved the step
    // loop's schedule and cost 4%, so there the compiler places those loads.
    if constexpr (D == 128) {
        pin_args(a.dO);
        pin_args(a.lse);
        pin_args(a.delta);
        pin_args(a.do_absmax);
        pin_args(a.dk);
        pin_args(a.dv);
        pin_args(a.dkv_rs);
    }
    using C = DkvCfg<D, BQ, NKW, HS, NR>;
    __shared__ __attribute__((aligned(1024))) char smem[C::kLds];
    __shared__ unsigned wg_red[C::kThreads / 64];   // one word per wave: the dO scale search
    __shared__ float sigma_sh;                      // the dO scale (see below)

    const int T = a.T, Hq = a.Hq, Hkv = a.Hkv;
    const int G = a.div.G;
    const int bg_count = a.B * Hkv;
    const int bid = blockIdx.x;
    const int kt = udiv(bid, a.div.bhkv);          // which group of block positions
    const int bg = bid - kt * bg_count;
    const int b = udiv(bg, a.div.hkv), g = bg - b * Hkv;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int hs = wave / NKW;                     // head slot
    const int kwr = wave % NKW;                    // wave index within the slot
    const int pos = (kwr + hs) % NKW;              // key-block position within the workgroup
    const int stid = tid % C::kSlotThreads;        // thread index within the slot
    const int n = lane & 31, hl = lane >> 5;
    // Workgroup kt takes positions NKW*kt .. NKW*kt + NKW - 1 of the block order: the
    // identity, or zig-zag (position p holds block p/2 for even p, nkb - 1 - p/2 for
    // odd p). Either way its earliest block sits at its first position.
    const int nkb = (T + 31) / 32;
    auto block_at = [&](int p) { return !a.zigzag ? p : (p & 1) ? nkb - 1 - (p >> 1) : (p >> 1); };
    const int p0 = NKW * kt;
    const int kb_first = p0 < nkb ? block_at(p0) : nkb;   // the workgroup's earliest block
    const int gp = p0 + pos;
    const int kwb = gp < nkb ? 32 * block_at(gp) : T;     // first key of this wave (T: none)
    const int key = kwb + n;                       // this lane's key (column)

    // Steps of a slot: its heads ascending, then query tiles ascending from the tile
    // holding the workgroup's earliest key. Every slot has the same number of steps
    // (HS divides G).
    const int nqt = (T + BQ - 1) / BQ;
    const int qt_begin = (32 * kb_first) / BQ;
    const int per_head = nqt - qt_begin;
    const int heads_per_slot = G / HS;
    const int nsteps = kb_first < nkb ? heads_per_slot * per_head : 0;

    char* slot_base = smem + hs * C::kSlot;
    auto conv_stage = [&](int st) { return slot_base + NR * C::kRawStage + (st & 1) * C::kConvStage; };
    // A step's head, first query and raw ring stage, advanced one step at a time (the
    // DMA and the conversion each keep one, for the next step they handle).
    struct Cursor {
        int h, q0, stage;
        size_t row, row_do;   // element offsets of the step's first Q and dO rows
        size_t stat;          // element offset of the step's first lse / delta value
    };
    auto head_start = [&](Cursor& c, int h) CGQA_INLINE {
        c.h = h;
        c.q0 = qt_begin * BQ;
        c.row = ((size_t)b * T + c.q0) * a.q_rs + (size_t)h * D;
        if constexpr (!SAME_QDO) c.row_do = ((size_t)b * T + c.q0) * a.do_rs + (size_t)h * D;
        c.stat = ((size_t)b * Hq + h) * T + c.q0;
    };
    auto advance = [&](Cursor& c) CGQA_INLINE {
        c.q0 += BQ;
        c.row += (size_t)BQ * a.q_rs;
        if constexpr (!SAME_QDO) c.row_do += (size_t)BQ * a.do_rs;
        c.stat += BQ;
        if (c.q0 >= nqt * BQ) head_start(c, c.h + HS);
        c.stage = c.stage + 1 == NR ? 0 : c.stage + 1;
    };
    Cursor dma_cur;
    dma_cur.stage = 0;
    head_start(dma_cur, g * G + hs);
    Cursor cvt_cur = dma_cur;

    // DMA of one step into the raw ring: each wave of the slot copies kTileLoads KB of
    // Q rows and of dO rows (row-major, 1 KB per instruction), and kStatLanes floats of
    // lse / delta (4 bytes per lane), from a wave-uniform base (the step's first row)
    // plus constant lane offsets. Query rows past T read row T-1; the conversion masks
    // them.
    const unsigned lds0 = __builtin_amdgcn_readfirstlane(
        (unsigned)(uintptr_t)(const __attribute__((address_space(3))) char*)smem);
    const unsigned q_row_bytes = (unsigned)a.q_rs * 2u, do_row_bytes = (unsigned)a.do_rs * 2u;
    int dma_row[C::kTileLoads];
    unsigned dma_col[C::kTileLoads], dma_off[C::kTileLoads], dma_off_do[C::kTileLoads];
#pragma unroll
    for (int i = 0; i < C::kTileLoads; ++i) {
        const int byte = (kwr * C::kTileLoads + i) * 1024 + 16 * lane;
        dma_row[i] = byte / C::kRawRow;
        dma_col[i] = (unsigned)(byte % C::kRawRow);
        dma_off[i] = (unsigned)dma_row[i] * q_row_bytes + dma_col[i];
        dma_off_do[i] = SAME_QDO ? dma_off[i] : (unsigned)dma_row[i] * do_row_bytes + dma_col[i];
    }
    const bool stat_lse = kwr * C::kStatLanes < BQ;          // wave-uniform: lse or delta
    const int stat_row = (kwr * C::kStatLanes + lane) % BQ;
    auto issue_step = [&]() CGQA_INLINE {
        const unsigned raw = lds0 + (unsigned)(slot_base - smem) + dma_cur.stage * C::kRawStage;
        const int qs0 = dma_cur.q0;
        const int last = T - 1 - qs0;                        // rows past it repeat row T-1
        unsigned off[C::kTileLoads], off_do[C::kTileLoads];
        if (qs0 + BQ <= T) {
#pragma unroll
            for (int i = 0; i < C::kTileLoads; ++i) {
                off[i] = dma_off[i];
                off_do[i] = SAME_QDO ? dma_off[i] : dma_off_do[i];
            }
        } else {
#pragma unroll
            for (int i = 0; i < C::kTileLoads; ++i) {
                const unsigned r = (unsigned)min(dma_row[i], last);
                off[i] = r * q_row_bytes + dma_col[i];
                off_do[i] = SAME_QDO ? off[i] : r * do_row_bytes + dma_col[i];
            }
        }
        // One instruction per chunk, each with its own (never negative) lane offset: the
        // 32-bit offset is zero-extended, so an offset reduced by a later chunk's
        // instruction offset could wrap when a ragged tile clamps its rows.
        const unsigned lds = raw + kwr * C::kTileLoads * 1024;
#pragma unroll
        for (int i = 0; i < C::kTileLoads; ++i) {
            const unsigned o1[1] = {off[i]}, o2[1] = {off_do[i]};
            load_lds16_chunks<1>(a.q + dma_cur.row, o1, lds + 1024 * i);
            load_lds16_chunks<1>(a.dO + (SAME_QDO ? dma_cur.row : dma_cur.row_do), o2, lds + C::kRawTile + 1024 * i);
        }
        if constexpr (C::kStatLoads == 2) {
            // Lanes 0 .. BQ-1 take lse, the others delta; both halves are always active.
            const unsigned so = (unsigned)min(stat_row, last) * 4u, sd = raw + 2 * C::kRawTile;
            if (lane < BQ) load_lds4_off(a.lse + dma_cur.stat, so, sd);
            else load_lds4_off(a.delta + dma_cur.stat, so, sd);
        } else if (lane < C::kStatLanes) {
            const float* sb = (stat_lse ? a.lse : a.delta) + dma_cur.stat;
            load_lds4_off(sb, (unsigned)min(stat_row, last) * 4u, raw + 2 * C::kRawTile + kwr * C::kStatLanes * 4);
        }
        advance(dma_cur);
    };
    // dO (and with it dP, delta and dS) is multiplied by the workgroup's power-of-two scale
    // sigma before its fp16 rounding; dK and dV are multiplied back by 1 / sigma at the
    // store (see the header). The loop reads sigma from LDS at each conversion instead of
    // keeping it in a register: the loop sits at the register budget of three waves per
    // SIMD, and one more live value there makes the compiler trade the products'
    // overlap with the softmax for register pressure (measured: about 7% slower).
    auto load_sigma = [&]() CGQA_INLINE {
        return __uint_as_float(__builtin_amdgcn_readfirstlane(__float_as_uint(sigma_sh)));   // uniform: a scalar
    };
    // Raw step -> converted step (fp16 rows, scaled and masked statistics). `idle` is the
    // set of the slot's waves (bit kwr) that have no products in the current step: when
    // there are some, they do the whole conversion between them and the waves with
    // products skip it; otherwise every thread of the slot converts its share. (A slot's
    // late key blocks wait for most of the stream before their diagonal comes.) Both
    // ways give the same bits. At d = 128 (one wave per SIMD at 256 registers) the extra
    // path made the loop slower; there every thread converts its share.
    constexpr bool kIdleConvert = D == 64;
    auto convert_chunk = [&](const char* raw, char* cv, int t, int ch, float sigma) CGQA_INLINE {
        const int row = ch / (C::kRawRow / 16), col = ch % (C::kRawRow / 16);
        const u32x4 x = *reinterpret_cast<const u32x4*>(raw + t * C::kRawTile + ch * 16);
        store16(cv + t * C::kTile + row * C::kPitch + col * 16,
                t == 0 ? bf16x8_to_f16_bits(x) : bf16x8_to_f16_bits_scaled(x, sigma));
    };
    auto convert_stat = [&](const char* raw, char* cv, int i, int qs0, float sigma) CGQA_INLINE {
        const float x = reinterpret_cast<const float*>(raw + 2 * C::kRawTile)[i];
        const bool valid = qs0 + (i % BQ) < T;
        float y;
        if (i < BQ) y = valid ? x * kLog2e : INFINITY;    // P = 0 past T
        else y = valid ? x * sigma : 0.0f;
        reinterpret_cast<float*>(cv + 2 * C::kTile)[i] = y;
    };
    auto convert_step = [&](int st, float sigma, unsigned idle) CGQA_INLINE {
        const char* raw = slot_base + cvt_cur.stage * C::kRawStage;
        char* cv = conv_stage(st);
        const int qs0 = cvt_cur.q0;
        advance(cvt_cur);
        if (!kIdleConvert || idle == 0) {
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int i = 0; i < C::kConvChunks; ++i) convert_chunk(raw, cv, t, stid + i * C::kSlotThreads, sigma);
            if (stid < 2 * BQ) convert_stat(raw, cv, stid, qs0, sigma);
        } else if (idle >> kwr & 1u) {
            constexpr int kPerTensor = C::kRawTile / 16;
            const int nid = __builtin_popcount(idle);
            const int rank = __builtin_popcount(idle & ((1u << kwr) - 1u));
            for (int ch = 64 * rank + lane; ch < kPerTensor; ch += 64 * nid) convert_chunk(raw, cv, 0, ch, sigma);
            for (int ch = 64 * rank + lane; ch < kPerTensor; ch += 64 * nid) convert_chunk(raw, cv, 1, ch, sigma);
            if (rank == 0 && lane < 2 * BQ) convert_stat(raw, cv, lane, qs0, sigma);
        }
    };
    auto wait_barrier = [&](int pending_steps) CGQA_INLINE {
        // pending_steps: how many of this wave's issued steps may still be in flight.
        if (pending_steps <= 0) wait_tiles_barrier<0>();
        else if (pending_steps == 1) wait_tiles_barrier<C::kVmPerStep>();
        else wait_tiles_barrier<2 * C::kVmPerStep>();
    };

    // Prologue: DMA step 0, then load K and V of the lane's key as B operands (dims
    // 16*kd + 8*hl .. +7) in fp16, and the dO block maxima of the group, so the
    // latencies overlap; only these are waited for before the later steps are issued.
    if (nsteps > 0) issue_step();
    // The scale: the largest |dO| over every query row of the group's heads (published
    // by attn_bwd_dq per block of 32 rows; non-negative floats, so their bit patterns
    // order like the values), into [1, 2). Every workgroup of a (batch, kv head) group
    // gets the same scale, whatever the grid.
    {
        const int nblk = (T + 31) / 32;
        const float* am = a.do_absmax + ((size_t)b * Hq + (size_t)g * G) * nblk;
        unsigned bits = 0;
        for (int i = tid; i < G * nblk; i += C::kThreads) bits = max(bits, __float_as_uint(am[i]) >> 16);
        const unsigned wmax = wave_max_u32(bits);
        if (lane == 0) wg_red[wave] = wmax;
    }
    f16x8 kreg[C::kKD], vreg[C::kKD];
#pragma unroll
    for (int kd = 0; kd < C::kKD; ++kd) {
        u32x4 xk = {0u, 0u, 0u, 0u}, xv = {0u, 0u, 0u, 0u};
        if (key < T) {
            const size_t off = ((size_t)b * T + key) * a.kv_rs + (size_t)g * D + 16 * kd + 8 * hl;
            xk = load16(a.k + off);
            xv = load16(a.v + off);
        }
        kreg[kd] = bf16x8_to_f16(xk);
        vreg[kd] = bf16x8_to_f16(xv);
    }
    // K and V in registers before the loop on every path, so the compiler's waits for
    // them stay out of the loop (there they would also wait for the DMA prefetch, which
    // the compiler does not track).
#pragma unroll
    for (int kd = 0; kd < C::kKD; ++kd) asm volatile("" ::"v"(kreg[kd]), "v"(vreg[kd]));

    f32x16 dkacc[C::kMB], dvacc[C::kMB];
#pragma unroll
    for (int mb = 0; mb < C::kMB; ++mb) { dkacc[mb] = zero16(); dvacc[mb] = zero16(); }

    wait_tiles_barrier<0>();
    {
        unsigned m = 0;
#pragma unroll
        for (int w = 0; w < C::kThreads / 64; ++w) m = max(m, wg_red[w]);
        const float sigma = pow2_normalizer(__builtin_amdgcn_readfirstlane(m)).s;
        if (tid == 0) sigma_sh = sigma;      // read in the loop, after its first barrier
        for (int st = 1; st < NR && st < nsteps; ++st) issue_step();
        if (nsteps > 0) convert_step(0, sigma, 0u);
    }

    const int tr_row = (lane & 15) >> 2;
    const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);

    // One 32-query block of a step against the wave's keys. The causal mask is needed
    // only on the wave's diagonal block (first query = first key): MASK is a
    // compile-time flag so that the other blocks carry no comparisons.
    auto block = [&](auto Mc, const char* qs, const char* ds, const float* lse2s, const float* dels, int sb) CGQA_INLINE {
        constexpr bool MASK = decltype(Mc)::value;
        f32x16 s = zero16(), dp = zero16();
#pragma unroll
        for (int kd = 0; kd < C::kKD; ++kd) {
            const int off = (32 * sb + n) * C::kPitch + (16 * kd + 8 * hl) * 2;
            s = mfma32x32x16(lds_read8_f16(qs + off), kreg[kd], s);
            dp = mfma32x32x16(lds_read8_f16(ds + off), vreg[kd], dp);
        }
        // Register i holds query 8*(i/4) + 4*hl + i%4 of the block, of the lane's key.
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int r = 32 * sb + 8 * u + 4 * hl;
            const f32x4 l4 = *reinterpret_cast<const f32x4*>(lse2s + r);
            const f32x4 d4 = *reinterpret_cast<const f32x4*>(dels + r);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int i = 4 * u + e;
                float p = exp2_fast(fmaf(s[i], a.scale_log2, -l4[e]));
                if constexpr (MASK)
                    if (n > 8 * u + 4 * hl + e) p = 0.0f;      // key after query
                s[i] = p;
                dp[i] = p * (dp[i] - d4[e]);           // dS
            }
        }
        // dV^T += dO^T P and dK^T += Q^T dS, 16 queries per instruction.
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const f16x8 pb = t == 0 ? pack_lo_f16(s) : pack_hi_f16(s);
            const f16x8 sb8 = t == 0 ? pack_lo_f16(dp) : pack_hi_f16(dp);
            const int r0 = 32 * sb + 16 * t + 4 * hl + tr_row;
#pragma unroll
            for (int mb = 0; mb < C::kMB; ++mb) {
                const int off = r0 * C::kPitch + (32 * mb + tr_col) * 2;
                const f16x8 dot = concat(lds_read_tr4_f16(ds + off), lds_read_tr4_f16(ds + off + 8 * C::kPitch));
                const f16x8 qt8 = concat(lds_read_tr4_f16(qs + off), lds_read_tr4_f16(qs + off + 8 * C::kPitch));
                dvacc[mb] = mfma32x32x16(dot, pb, dvacc[mb]);
                dkacc[mb] = mfma32x32x16(qt8, sb8, dkacc[mb]);
            }
        }
    };

    // Step `step` of the slot: wait for its data (and retire the stages that the next
    // DMA and conversion reuse) and start the DMA NR steps ahead. The next step is
    // converted after this step's products are issued (convert_next), so that the
    // conversion's LDS round trip overlaps the matrix core instead of delaying the
    // operand reads: its raw stage is complete at this barrier, its fp16 stage was
    // last read before it, and the next barrier publishes it.
    auto sync_step = [&](int step) CGQA_INLINE {
        // Step+1 complete in LDS (only newer steps may be in flight); the barrier also
        // retires every wave's use of the stages that the next DMA and conversion reuse.
        wait_barrier(min(step + NR - 1, nsteps - 1) - (step + 1));
        if (step + NR < nsteps) issue_step();
    };
    auto convert_next = [&](int step, unsigned idle) CGQA_INLINE {
        if (step + 1 < nsteps) convert_step(step + 1, load_sigma(), idle);
    };
    auto compute_step = [&](auto Mc, int step) CGQA_INLINE {
        const char* qs = conv_stage(step);
        const char* ds = qs + C::kTile;
        const float* lse2s = reinterpret_cast<const float*>(ds + C::kTile);
        block(Mc, qs, ds, lse2s, lse2s + BQ, 0);
    };
    // Each head pass of the slot: the steps before the wave's diagonal block (queries
    // that precede all its keys: loads and conversions only), the diagonal step (with
    // the mask), then the rest. Waves without a block only keep the loads going.
    const int diag = kwb < T ? kwb / 32 - qt_begin : per_head;   // diagonal step within a pass
    // The diagonal steps of the slot's waves (wave kwr of slot hs holds position
    // (kwr + hs) % NKW): wave k has no products in the steps of a pass before its own.
    int slot_diag[NKW];
#pragma unroll
    for (int k = 0; k < NKW; ++k) {
        const int gpk = p0 + (k + hs) % NKW;
        slot_diag[k] = gpk < nkb ? block_at(gpk) - qt_begin : per_head;
    }
    auto idle_at = [&](int r) CGQA_INLINE {   // r: step within the pass
        unsigned m = 0;
#pragma unroll
        for (int k = 0; k < NKW; ++k) m |= (r < slot_diag[k] ? 1u : 0u) << k;
        return m;
    };
    for (int hp = 0; hp < heads_per_slot; ++hp) {
        const int s0 = hp * per_head, s1 = s0 + per_head;
        const int sd = min(s0 + diag, s1);
        int step = s0;
        for (; step < sd; ++step) {
            sync_step(step);
            convert_next(step, idle_at(step - s0));
        }
        if (step < s1) {
            sync_step(step);
            compute_step(std::true_type{}, step);
            convert_next(step, idle_at(step - s0));
            ++step;
        }
        for (; step < s1; ++step) {
            sync_step(step);
            compute_step(std::false_type{}, step);
            convert_next(step, idle_at(step - s0));
        }
    }
    lds_barrier();

    // ---- sum the head slots (ascending) and store: one 32-dim block of dK, then of dV,
    // at a time through the same LDS area; every wave's lane values line up across
    // slots. A wave's block is stored as four groups of 64 lanes x 16 bytes, so each
    // 16-byte access of a wave covers 1 KB of consecutive LDS (no bank conflicts).
    float* red = reinterpret_cast<float*>(smem);
    auto red_at = [&](int slot, int u) { return red + (size_t)((((slot - 1) * NKW + pos) * 4 + u) * 64 + lane) * 4; };
    // Rotary tables of this lane's key (clamped in range for lanes without one), loaded
    // together before the reduction, by the waves that store, so their latency is paid
    // once.
    RopeCS rt[C::kMB][4];
    if constexpr (ROPE) {
        if (hs == 0) {   // only head slot 0 stores
        const int kt_row = min(key, T - 1);
#pragma unroll
        for (int mb = 0; mb < C::kMB; ++mb)
#pragma unroll
            for (int u = 0; u < 4; ++u) rt[mb][u] = rope_load(a.rope_cos, a.rope_sin, kt_row, D / 2, 32 * mb + 8 * u + 4 * hl);
        }
    }
    auto reduce_store = [&](f32x16 (&acc)[C::kMB], void* out, float mul, auto Rc) {
        constexpr bool ROT = decltype(Rc)::value;
#pragma unroll
        for (int mb = 0; mb < C::kMB; ++mb) {
            if (HS > 1) {
                if (hs > 0) {
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        f32x4 x;
#pragma unroll
                        for (int r = 0; r < 4; ++r) x[r] = acc[mb][4 * u + r];
                        *reinterpret_cast<f32x4*>(red_at(hs, u)) = x;
                    }
                }
                lds_barrier();
                if (hs == 0) {
#pragma unroll
                    for (int s2 = 1; s2 < HS; ++s2) {
#pragma unroll
                        for (int u = 0; u < 4; ++u) {
                            const f32x4 x = *reinterpret_cast<const f32x4*>(red_at(s2, u));
#pragma unroll
                            for (int r = 0; r < 4; ++r) acc[mb][4 * u + r] += x[r];
                        }
                    }
                }
                lds_barrier();
            }
            if (hs == 0 && key < T) {
                const size_t row = ((size_t)b * T + key) * a.dkv_rs + (size_t)g * D;
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    f32x4 x;
#pragma unroll
                    for (int r = 0; r < 4; ++r) x[r] = acc[mb][4 * u + r] * mul;
                    if constexpr (ROT) x = rope_back4(x, rt[mb][u]);
                    store_out4(out, row + 32 * mb + 8 * u + 4 * hl, x, BF16OUT);
                }
            }
        }
    };
    // 1 / sigma for a power of two 2^k (k in [-126, 126]): exponent field 254 - that of sigma
    const float sigma_inv = __uint_as_float((254u << 23) - __float_as_uint(load_sigma()));
    reduce_store(dkacc, a.dk, a.scale * sigma_inv, std::integral_constant<bool, ROPE>{});
    reduce_store(dvacc, a.dv, sigma_inv, std::false_type{});
}

// ---- Software-pipelined dQ (d = 64) ---------------------------------------------------
//
// Workgroup: 4 waves x 32 queries of one head; a step is one 32-key block. In step t a
// wave issues dQ~ += K^T dS~(t-1) and K_bar += K^T P(t-1) on the fp16 matrix core while
// its vector ALU turns block t into P, dS~ and the exact D, then issues S^T(t+1) = K Q^T
// and dP^T(t+1) = V dO^T on the bf16 matrix core (inputs straight from the raw tiles:
// bf16 products are exact in fp32) into the registers block t just released. Raw K and V arrive by direct-to-LDS loads in a 4-stage ring
// (3 steps ahead); K is also converted once to fp16 into a 4-slot padded ring for the
// transposing reads. K(u) is read raw in step u-1 (scores, conversion) and in fp16 in
// step u+1; V(u) in step u-1.
template <int D>
struct DqPipeCfg {
    static constexpr int kNW = 4;
    static constexpr int kThreads = 64 * kNW;
    static constexpr int kBM = 32 * kNW;             // queries per workgroup
    static constexpr int kKD = D / 16;
    static constexpr int kMB = D / 32;
    static constexpr int kRow = 2 * D;               // raw bf16 row (swizzled chunks)
    static constexpr int kTile = 32 * kRow;          // raw K (or V) of a 32-key block
    static constexpr int kRawStage = 2 * kTile;      // K then V
    static constexpr int kDepth = 4;
    static constexpr int kRaw = kDepth * kRawStage;
    static constexpr int kHalfTile = 32 * kRow;      // fp16 K of a block (swizzled chunks, as the raw tiles)
    static constexpr int kLds = kRaw + kDepth * kHalfTile;
    static constexpr int kChunks = kTile / 1024;     // 1 KB DMA chunks per tensor
    static constexpr int kRowsPerChunk = 1024 / kRow;
    static_assert(kChunks == kNW, "one K and one V chunk per wave and step");
    static_assert(kLds <= 160 * 1024, "LDS budget");
};

template <int D>
__global__ __launch_bounds__(256, 2) void attn_bwd_dq_pipe_kernel(BwdArgs a_in) {
    BwdArgs a = a_in;
    pin_args(a);   // all argument loads at entry (see pin_args)
    using C = DqPipeCfg<D>;
    __shared__ __attribute__((aligned(1024))) char smem[C::kLds];
    char* const raw = smem;
    char* const k16 = smem + C::kRaw;

    // Workgroup-uniform indices (readfirstlane keeps the integer divisions' results,
    // and everything derived from them, in scalar registers).
    const int T = a.T, Hq = a.Hq;
    const DqTile wg = dq_tile(a, blockIdx.x);
    const int qt = __builtin_amdgcn_readfirstlane(wg.qt);   // heaviest first
    const int b = __builtin_amdgcn_readfirstlane(wg.b);
    const int h = __builtin_amdgcn_readfirstlane(wg.h);
    const int g = __builtin_amdgcn_readfirstlane(udiv(h, a.div.g));

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n = lane & 31, hl = lane >> 5;
    const int q0 = qt * C::kBM;
    const int qw = q0 + 32 * wave;                    // first query of this wave
    const int nb_wg = (min(T, q0 + C::kBM) + 31) / 32; // key blocks the workgroup needs
    const int my_n = (qw < T) ? qw / 32 + 1 : 0;      // key blocks of this wave

    const uint16_t* kbase = a.k + (size_t)b * T * a.kv_rs + (size_t)g * D;
    const uint16_t* vbase = a.v + (size_t)b * T * a.kv_rs + (size_t)g * D;
    const unsigned kv_row_bytes = (unsigned)a.kv_rs * 2u;

    // DMA: wave w loads chunk w (rows 8w .. 8w+7 for D = 64) of K and of V of a block.
    // Blocks outside 0 .. nb_wg-1 reload the last block (into a stage nobody reads), so
    // every step issues the same two full-wave loads and the waits are constants. In the
    // last block of a ragged sequence, rows past T repeat row T-1 (finite data; those
    // keys are masked for every real query).
    const int ld_r = C::kRowsPerChunk * wave + lane / (C::kRow / 16);
    const unsigned voff = (unsigned)ld_r * kv_row_bytes +
                          (unsigned)((lane % (C::kRow / 16)) ^ chunk_swizzle<D>(ld_r)) * 16u;
    const unsigned lds0 = __builtin_amdgcn_readfirstlane(
        (unsigned)(uintptr_t)(const __attribute__((address_space(3))) char*)smem);
    auto issue = [&](int stage, int u) {
        const int uc = min(max(u, 0), nb_wg - 1);
        const int rows = T - 32 * uc;
        const unsigned lds = lds0 + stage * C::kRawStage + wave * 1024;
        const char* kb = reinterpret_cast<const char*>(kbase) + (size_t)(32 * uc) * kv_row_bytes;
        const char* vb = reinterpret_cast<const char*>(vbase) + (size_t)(32 * uc) * kv_row_bytes;
        const unsigned o[1] = {rows >= 32 ? voff
                                          : (unsigned)min(ld_r, rows - 1) * kv_row_bytes +
                                                (unsigned)((lane % (C::kRow / 16)) ^ chunk_swizzle<D>(ld_r)) * 16u};
        load_lds16_chunks<1>(kb, o, lds);
        load_lds16_chunks<1>(vb, o, lds + C::kTile);
    };
#pragma unroll
    for (int u = 0; u < 3; ++u) issue(u, u);   // what steps -4 .. -2 issue

    // Q, dO (bf16, as given) as B operands (lane: query n, dims 16*kd + 8*hl .. +7),
    // D~ = rowsum(dO * O) from the given bf16 O, and the row's LSE in log2 units.
    bf16x8 qreg[C::kKD], doreg[C::kKD];
    float dtilde, lse2, dexact = 0.0f, dsc, dsc_inv, dts;
    {
        const int row = qw + n;
        float part = 0.0f;
        unsigned dmax = 0;
#pragma unroll
        for (int kd = 0; kd < C::kKD; ++kd) {
            u32x4 xq = {0u, 0u, 0u, 0u}, xd = {0u, 0u, 0u, 0u}, xo = {0u, 0u, 0u, 0u};
            if (row < T) {
                const size_t rowg = (size_t)b * T + row;
                const int col = h * D + 16 * kd + 8 * hl;
                xq = load16(a.q + rowg * a.q_rs + col);
                xd = load16(a.dO + rowg * a.do_rs + col);
                xo = load16(a.o + rowg * a.o_rs + col);
            }
            qreg[kd] = __builtin_bit_cast(bf16x8, xq);
            doreg[kd] = __builtin_bit_cast(bf16x8, xd);
            dmax = max(dmax, bf16x8_absmax_bits(xd));
            const bf16x8 dv8 = __builtin_bit_cast(bf16x8, xd);
            const bf16x8 ov8 = __builtin_bit_cast(bf16x8, xo);
#pragma unroll
            for (int e = 0; e < 8; ++e) part += (float)dv8[e] * (float)ov8[e];
        }
        part += swap_halves(part);
        dtilde = part;
        // dS of this row is scaled by 2^k (largest |dO| of the row into [1, 2)) before its
        // fp16 rounding, and dQ~ scaled back at the store.
        dmax = max(dmax, (unsigned)__shfl_xor((int)dmax, 32, 64));
        // The block's largest |dO| (its 32 rows), published for the dK/dV pass.
        const unsigned bmax = wave_max_u32(dmax);
        if (lane == 0 && qw < T) a.do_absmax[((size_t)b * Hq + h) * ((T + 31) / 32) + qw / 32] = __uint_as_float(bmax << 16);
        const Pow2Scale ps = pow2_normalizer(dmax);
        dsc = ps.s;
        dsc_inv = ps.inv;
        dts = part * ps.s;
        lse2 = row < T ? a.lse[((size_t)b * Hq + h) * T + row] * kLog2e : 0.0f;
#pragma unroll
        for (int kd = 0; kd < C::kKD; ++kd) asm volatile("" ::"v"(qreg[kd]), "v"(doreg[kd]));
    }

    f32x16 dqacc[C::kMB], kbar[C::kMB];
#pragma unroll
    for (int mb = 0; mb < C::kMB; ++mb) { dqacc[mb] = zero16(); kbar[mb] = zero16(); }
    // S^T and dP^T of the block being turned into probabilities, and the fp16 P and
    // dS~ (two B operands each) of the previous block: the products of block t-1 are
    // issued (and read their operands) before block t's softmax overwrites them.
    f32x16 sc = zero16(), dpc = zero16();
    f16x8 pk[2] = {f16x8{}, f16x8{}}, dsk[2] = {f16x8{}, f16x8{}};

    // Per-lane LDS addresses. A operand rows (raw tile): row n, logical chunk 2kd + hl.
    // Transposing reads of fp16 K: rows 16tt + 4hl + (lane&15)/4 (+8), columns
    // 32mb + 16((lane>>4)&1) + 4(lane&3), i.e. logical chunk 4mb + 2((lane>>4)&1) +
    // (lane&3)/2, 8 bytes in. The fp16 tile has the raw tiles' chunk swizzle (a padded
    // pitch lets the four rows of a transposing read meet in the same banks); rows enter
    // it through r % 16, so 16tt is an immediate.
    const char* aaddr[C::kKD];
    {
        const int swz = chunk_swizzle<D>(n);
#pragma unroll
        for (int kd = 0; kd < C::kKD; ++kd) aaddr[kd] = raw + n * C::kRow + (((2 * kd + hl) ^ swz) << 4);
    }
    const char* traddr[C::kMB][2];
    {
        const int r0 = 4 * hl + ((lane & 15) >> 2);
        const int chunk = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
#pragma unroll
        for (int mb = 0; mb < C::kMB; ++mb)
#pragma unroll
            for (int r = 0; r < 2; ++r)
                traddr[mb][r] = k16 + (r0 + 8 * r) * C::kRow + 8 * (lane & 1) +
                                (((4 * mb + chunk) ^ chunk_swizzle<D>(r0 + 8 * r)) << 4);
    }
    // Conversion of a raw K block to fp16: thread tid takes row tid/8, logical chunk tid%8.
    const int cv_r = tid / (C::kRow / 16), cv_c = tid % (C::kRow / 16);
    const char* cv_src = raw + cv_r * C::kRow + ((cv_c ^ chunk_swizzle<D>(cv_r)) << 4);
    char* cv_dst = k16 + cv_r * C::kRow + ((cv_c ^ chunk_swizzle<D>(cv_r)) << 4);

    // (ALWAYS: the caller knows block t+1 exists.)
    auto sync_and_stage = [&](int t, int iss, int rst, int cst, auto Ac) {
        // Loads of steps t-2 and t-1 (two per wave and step) may stay in flight; the
        // older ones hold K(t+1) and V(t+1).
        wait_tiles_barrier<4>();
        issue(iss, t + 4);                    // into the stage K(t), V(t) left
        if (decltype(Ac)::value || t + 1 < nb_wg) {
            const u32x4 x = __builtin_bit_cast(u32x4, lds_read8(cv_src + rst * C::kRawStage));
            store16(cv_dst + cst * C::kHalfTile, bf16x8_to_f16_bits(x));
        }
    };
    // Scores and dP of block t+1 (bf16 matrix core).
    auto mfma_sdp = [&](int rst, f32x16& sn, f32x16& dpn) {
        bf16x8 ka[C::kKD], va[C::kKD];
#pragma unroll
        for (int kd = 0; kd < C::kKD; ++kd) {
            ka[kd] = lds_read8(aaddr[kd] + rst * C::kRawStage);
            va[kd] = lds_read8(aaddr[kd] + rst * C::kRawStage + C::kTile);
        }
        sn = zero16();
        dpn = zero16();
#pragma unroll
        for (int kd = 0; kd < C::kKD; ++kd) {
            sn = mfma32x32x16(ka[kd], qreg[kd], sn);
            dpn = mfma32x32x16(va[kd], doreg[kd], dpn);
        }
    };
    // P, dS~ and D of block t; the mask only on the wave's diagonal block.
    // (In place: the scores become P, dP becomes dS~; both are dead afterwards.)
    // The steady steps never meet the diagonal and take MAY_MASK = false: a run-time
    // test alone would be if-converted and the comparisons executed on every block.
    auto softmax = [&](auto Mc, int t, f32x16& sc, f32x16& dpc, f16x8 (&pk)[2], f16x8 (&dk)[2]) {
        constexpr bool MAY_MASK = decltype(Mc)::value;
        const bool diag = t == my_n - 1;
        const int rel = 32 * t + 4 * hl - (qw + n);   // key - query at i = 0
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            float e = exp2_fast(fmaf(sc[i], a.scale_log2, -lse2));
            if constexpr (MAY_MASK)
                if (diag && rel + 8 * (i >> 2) + (i & 3) > 0) e = 0.0f;
            dexact = fmaf(e, dpc[i], dexact);
            dpc[i] = e * fmaf(dpc[i], dsc, -dts);
            sc[i] = e;
        }
        pk[0] = pack_lo_f16(sc);
        pk[1] = pack_hi_f16(sc);
        dk[0] = pack_lo_f16(dpc);
        dk[1] = pack_hi_f16(dpc);
    };
    // dQ~^T += K^T dS~^T and K_bar^T += K^T P^T for block t-1 (fp16 matrix core).
    auto mfma_dq = [&](int cst, const f16x8 (&pk)[2], const f16x8 (&dk)[2]) {
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
#pragma unroll
            for (int mb = 0; mb < C::kMB; ++mb) {
                const int off = cst * C::kHalfTile + 16 * tt * C::kRow;
                const f16x8 kt = concat(lds_read_tr4_f16(traddr[mb][0] + off), lds_read_tr4_f16(traddr[mb][1] + off));
                dqacc[mb] = mfma32x32x16(kt, dk[tt], dqacc[mb]);
                kbar[mb] = mfma32x32x16(kt, pk[tt], kbar[mb]);
            }
        }
    };

    // Edge steps with run-time stages (P: parity of t).
    auto edge_step = [&](int t) {
        sync_and_stage(t, (t + 4) & 3, (t + 1) & 3, (t + 1) & 3, std::false_type{});
        if (t >= 1 && t - 1 < my_n) mfma_dq((t + 3) & 3, pk, dsk);
        if (t >= 0 && t < my_n) softmax(std::true_type{}, t, sc, dpc, pk, dsk);
        if (t + 1 < my_n) mfma_sdp((t + 1) & 3, sc, dpc);
    };
    edge_step(-1);
    edge_step(0);
    // Steady steps t = 1 .. my_n-2 in whole groups of four: copy U of a group handles
    // t = 4k + 1 + U, with raw stage and conversion slot (2 + U) % 4 for block t+1,
    // fp16 slot U % 4 for block t-1 and DMA stage (1 + U) % 4 known at compile time.
    // No copy leaves the loop early, so the accumulators stay in the same registers
    // across the copies; the 0-3 remaining steady steps take the run-time path.
    const int n_groups = max(0, my_n - 2) / 4;
    for (int k = 0; k < n_groups; ++k) {
        static_for<4>([&](auto Uc) {
            constexpr int U = decltype(Uc)::value;
            const int t = 4 * k + 1 + U;
            sync_and_stage(t, (1 + U) % 4, (2 + U) % 4, (2 + U) % 4, std::true_type{});
            mfma_dq(U % 4, pk, dsk);
            softmax(std::false_type{}, t, sc, dpc, pk, dsk);
            mfma_sdp((2 + U) % 4, sc, dpc);
        });
    }
    for (int t = 4 * n_groups + 1; t <= my_n - 2; ++t) edge_step(t);
    // The wave's last two steps with work, then the workgroup's remaining steps (loads
    // and conversions for the other waves).
    const int t_last = max(1, my_n - 1);
    edge_step(t_last);
    edge_step(t_last + 1);
    for (int t = t_last + 2; t <= nb_wg; ++t) sync_and_stage(t, (t + 4) & 3, (t + 1) & 3, (t + 1) & 3, std::false_type{});

    const int query = qw + n;
    const float dfull = dexact + swap_halves(dexact);
    if (query < T) {
        if (hl == 0) a.delta[((size_t)b * Hq + h) * T + query] = dfull;
        const float corr = dfull - dtilde;
        const size_t drow = ((size_t)b * T + query) * a.dq_rs + (size_t)h * D;
        // Rotary tables of this row, all loaded before the first store.
        RopeCS rt[C::kMB][4];
        if (a.rope_cos) {
#pragma unroll
            for (int mb = 0; mb < C::kMB; ++mb)
#pragma unroll
                for (int u = 0; u < 4; ++u) rt[mb][u] = rope_load(a.rope_cos, a.rope_sin, query, D / 2, 32 * mb + 8 * u + 4 * hl);
        }
#pragma unroll
        for (int mb = 0; mb < C::kMB; ++mb)
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                f32x4 x;
#pragma unroll
                for (int r = 0; r < 4; ++r) x[r] = a.scale * fmaf(-corr, kbar[mb][4 * u + r], dqacc[mb][4 * u + r] * dsc_inv);
                if (a.rope_cos) x = rope_back4(x, rt[mb][u]);
                store_out4(a.dq, drow + 32 * mb + 8 * u + 4 * hl, x, a.grad_bf16);
            }
    }
}

template <int D>
static hipError_t launch_dq_pipe(const BwdArgs& a, hipStream_t stream) {
    using C = DqPipeCfg<D>;
    BwdArgs x = a;
    x.n_tiles = (a.T + C::kBM - 1) / C::kBM;
    x.xcd_group = (a.B * a.Hkv) % 8 == 0 ? 1 : 0;
    const long blocks = (long)x.n_tiles * a.B * a.Hq;
    hipLaunchKernelGGL((attn_bwd_dq_pipe_kernel<D>), dim3((unsigned)blocks), dim3(C::kThreads), 0, stream, x);
    return hipGetLastError();
}

template <int D, int NQB, int BN, int NW>
static hipError_t launch_dq_t(const BwdArgs& a, hipStream_t stream) {
    using C = DqCfg<D, NQB, BN, NW>;
    BwdArgs x = a;
    x.n_tiles = (a.T + C::kBM - 1) / C::kBM;
    x.xcd_group = (a.B * a.Hkv) % 8 == 0 ? 1 : 0;
    const long blocks = (long)x.n_tiles * a.B * a.Hq;
    hipLaunchKernelGGL((attn_bwd_dq_kernel<D, NQB, BN, NW>), dim3((unsigned)blocks), dim3(C::kThreads), 0,
                       stream, x);
    return hipGetLastError();
}

template <int D, int BQ, int NKW, int HS, int NR>
static hipError_t launch_dkv_t(const BwdArgs& a, hipStream_t stream) {
    using C = DkvCfg<D, BQ, NKW, HS, NR>;
    BwdArgs x = a;
    x.n_tiles = ((a.T + 31) / 32 + NKW - 1) / NKW;
    const long blocks = (long)x.n_tiles * a.B * a.Hkv;
    // One workgroup per CU fits (LDS and registers); gfx950 parts have 256 CUs.
    x.zigzag = blocks <= 256 ? 1 : 0;
    const dim3 grid((unsigned)blocks), block(C::kThreads);
    const bool same = a.q_rs == a.do_rs;
    if (a.rope_cos) {
        // Rotary calls come contiguous (same Q and dO stride) with fp32 gradients.
        hipLaunchKernelGGL((attn_bwd_dkv_kernel<D, BQ, NKW, HS, NR, true, false, true>), grid, block, 0, stream, x);
    } else if (same && !a.grad_bf16)
        hipLaunchKernelGGL((attn_bwd_dkv_kernel<D, BQ, NKW, HS, NR, true, false, false>), grid, block, 0, stream, x);
    else if (same)
        hipLaunchKernelGGL((attn_bwd_dkv_kernel<D, BQ, NKW, HS, NR, true, true, false>), grid, block, 0, stream, x);
    else if (!a.grad_bf16)
        hipLaunchKernelGGL((attn_bwd_dkv_kernel<D, BQ, NKW, HS, NR, false, false, false>), grid, block, 0, stream, x);
    else
        hipLaunchKernelGGL((attn_bwd_dkv_kernel<D, BQ, NKW, HS, NR, false, true, false>), grid, block, 0, stream, x);
    return hipGetLastError();
}

hipError_t launch_bwd_dq(const BwdArgs& a, hipStream_t stream) {
    if (a.d == 64) return launch_dq_pipe<64>(a, stream);
    return launch_dq_t<128, 1, 32, 4>(a, stream);
}

// Head slots: as many as divide the group size and fit. A slot stages its own Q/dO
// tiles, and a workgroup of W waves keeps W/4 waves per SIMD, so the register budget of
// a wave bounds W: d=64 keeps up to 12 waves. A d=128 wave already needs all 256 VGPRs
// (extra slots spill), so d=128 uses one slot.
hipError_t launch_bwd_dkv(const BwdArgs& a, hipStream_t stream) {
    const int G = a.Hq / a.Hkv;
    if (a.d == 64) {
        if (G % 4 == 0) return launch_dkv_t<64, 32, 2, 4, 2>(a, stream);
        if (G % 3 == 0) {
            // Tiny grids (at most 32 workgroups of four key blocks) take one key block per
            // workgroup: four times the workgroups on an idle chip (B1 T64 Hq6 Hkv2: 9.1 ->
            // 7.2 us). Larger ones keep four: a single wave's step is no faster alone (B8
            // T512: 28.9 -> 30.5 us with one block per workgroup).
            const long nkb = (a.T + 31) / 32;
            if ((long)a.B * a.Hkv * ((nkb + 3) / 4) <= 32) return launch_dkv_t<64, 32, 1, 3, 3>(a, stream);
            return launch_dkv_t<64, 32, 4, 3, 3>(a, stream);
        }
        if (G % 2 == 0) return launch_dkv_t<64, 32, 4, 2, 3>(a, stream);
        return launch_dkv_t<64, 32, 4, 1, 3>(a, stream);
    }
    return launch_dkv_t<128, 32, 4, 1, 3>(a, stream);
}

}  // namespace cgqa
