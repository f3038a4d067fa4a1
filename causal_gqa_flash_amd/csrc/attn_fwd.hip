// Forward kernel of causal grouped-query flash attention for gfx950.
//
// Method (page "A transformer in PTX", section "Flash attention"): one workgroup owns
// a block of queries of one head and visits the key blocks from the first one to the
// block holding the diagonal. Scores never go to memory: each query carries a
// reference max m and a sum l (online softmax) in base-2 units, the scores being
// scaled a single time by scale * log2(e) and each probability being 2^(s - m). At the
// end O = acc / l, and the row's log-sum-exp, converted to natural log, is stored for
// the backward.
//
// gfx950 design (not the page's sm_120 one):
//  * The scores are computed transposed, S^T = K Q^T, on the 32x32x16 bf16 matrix
//    core. Each lane then owns one query (a column) and 16 keys of every 32-key block,
//    so a row reduction is an in-lane reduction plus one swap with the lane 32 away.
//  * The same accumulator registers, rounded to bf16, are the B operand of
//    O^T += V^T P^T: no trip through LDS for P (the role the pages give to their
//    C-fragment to A-fragment match). V^T comes from the row-major V tile through the
//    transposing LDS read.
//  * Software pipeline inside each wave. On gfx950 the vector ALU and the matrix core
//    only overlap well when one wave interleaves independent work for both; work of
//    two different waves on one SIMD mostly adds up. So the wave's step j issues the
//    scores of key block j+1 and the P.V product of block j-1 on the matrix core,
//    interleaved with the softmax of block j on the vector ALU (which depends on
//    neither). The diagonal block, the only masked one, is peeled off the loop.
//  * The reference max is not updated block by block. Softmax is invariant to the
//    reference (O = sum p v / sum p and LSE = m + log2 l hold for any m), so m is taken
//    from the first key block (which holds key 0 for every query) and kept while every
//    probability stays below 2^40. Only when a block's sum shows a larger value (a
//    score 40 log2 units above m) does the wave recompute that block's scores, move m
//    to the new row max and rescale l and the accumulators. This keeps the per-score
//    max and the per-block rescale off the vector ALU: one fma, one exp2, one add and
//    half a convert per score remain.
//  * K and V tiles go straight from global memory to LDS (global_load_lds_dwordx4, no
//    staging registers) into a ring of stages, 64 keys ahead of the compute; one
//    barrier per tile. A direct load writes 1 KB of consecutive LDS per instruction, so
//    rows cannot be padded; instead the 16-byte chunks of each row are XOR-swizzled
//    (see chunk_swizzle) so that both the 16-byte row reads of K and the transposing
//    reads of V spread over the 64 banks.
//  * Work order: workgroup x runs on XCD x mod 8. When the (batch, kv head) slices
//    split evenly over the XCDs, all query tiles of a slice go to one XCD, whose L2
//    then serves that slice's K and V to every query head of the group; on each XCD the
//    heaviest query tiles (the most keys) are dispatched first, or, when every
//    workgroup of the grid is resident from the start, in an order that gives each CU
//    about the same number of key blocks (balance_one_round: 4.5% faster at B16 T1024).
#include "cgqa_device.hpp"
#include "cgqa_launch.hpp"

#include <type_traits>

namespace cgqa {

template <int D, bool ROPE = false>
struct FwdCfg {
    // Query blocks of 32 per wave (the code also supports two, which halves the LDS
    // fragment reads per product but needs ~236 registers and so at most two waves per
    // SIMD; one block per wave allows three workgroups per CU at d = 64, which balances
    // the causal work better and measured faster).
    static constexpr int kNQB = 1;
    static constexpr int kWaves = 4;
    static constexpr int kThreads = 64 * kWaves;
    static constexpr int kWQ = 32 * kNQB;                   // queries per wave
    static constexpr int kBM = kWQ * kWaves;                // queries per workgroup
    // Keys per LDS tile: 64 at d = 64 (two 32-key blocks per barrier and per DMA batch,
    // three stages: 48 KB, three workgroups per CU; measured 0.3-8% faster than 32-key
    // tiles in five stages, except 2% slower at T = 4096), 32 at d = 128 (five stages:
    // 80 KB, two workgroups per CU). With the rotary embedding (ROPE, d = 64 only) the
    // tiles are 32 keys in five stages, 48 KB with the rotary tables.
    static constexpr int kBN = (D == 64 && !ROPE) ? 64 : 32;
    static constexpr int kBPT = kBN / 32;                   // 32-key blocks per tile
    static constexpr int kStages = (D == 64 && !ROPE) ? 3 : 5;
    // Tiles issued beyond the one a barrier waits for. At the barrier for tile t the
    // stage of tile t - 2 (kBPT = 2) or t - 3 (kBPT = 1) has been read for the last
    // time, which leaves kStages - 2 resp. kStages - 3 stages for tiles in flight.
    static constexpr int kAhead = kBPT == 2 ? kStages - 2 : kStages - 3;
    static constexpr int kKD = D / 16;                      // k-steps over the head dimension
    static constexpr int kMB = D / 32;                      // 32-dim blocks of the output
    static constexpr int kRow = D * 2;                      // bytes per K or V row in LDS
    static constexpr int kTile = kBN * kRow;                // bytes per K (or V) tile
    static constexpr int kStage = 2 * kTile;                // K then V
    static constexpr int kRing = kStages * kStage;
    static constexpr int kLoadsPerTensor = kTile / 1024 / kWaves;   // 1 KB per wave instruction
    static constexpr int kLoadsPerTile = 2 * kLoadsPerTensor;       // per wave
    static constexpr int kRowsPerLoad = 1024 / kRow;
    static constexpr int kUnroll = kStages * kBPT;          // period of the block -> stage map
    // ROPE: each thread's cosines and sines for the K chunks it loads (16 bytes of each
    // per chunk), by DMA into an area of its own after the ring.
    static constexpr int kTabHalf = ROPE ? kLoadsPerTensor * kWaves * 1024 : 0;
    static constexpr int kLds = kRing + 2 * kTabHalf;
    static_assert(D == 64 || D == 128, "head dim");
    static_assert(kTile % (1024 * kWaves) == 0, "tile load must split evenly over the waves");
    static_assert(kAhead * kBN >= 64, "prefetch distance: at least 64 keys in flight");
    // The rotary path turns each 32-key tile once (one block per tile) and exists at
    // d = 64 only: at d = 128 its extra registers would spill.
    static_assert(!ROPE || (kBPT == 1 && D == 64), "rotary configuration");
    static_assert(2 * kLds <= 160 * 1024, "two workgroups per CU");
    // Workgroups resident per CU: three at d = 64 (48 KB of LDS, at most 168 registers),
    // two at d = 128 (80 KB).
    static constexpr int kResident = D == 64 ? 3 : 2;
    static_assert(kResident * kLds <= 160 * 1024, "resident workgroups");
};

// Probabilities above this trigger a move of the reference max.
constexpr float kRescaleLimit = 1099511627776.0f;   // 2^40

template <int D, bool ROPE>
__global__ __launch_bounds__(256, D == 64 ? 3 : 2) void attn_fwd_kernel(FwdArgs a) {
    using C = FwdCfg<D, ROPE>;
    constexpr int NQB = C::kNQB;
    constexpr int kAll = (1 << NQB) - 1;   // bit qb: query block qb of the wave
    __shared__ __attribute__((aligned(1024))) char smem[C::kLds];

    const int T = a.T, Hq = a.Hq, Hkv = a.Hkv;
    const int G = a.div.G;
    int qt, b, h;
    if (a.xcd_group) {
        // Slices p = b * Hkv + g with p % 8 == x % 8 run on XCD x % 8 (n_pairs % 8 == 0).
        const int xcd = (int)blockIdx.x & 7;
        const int per_qt = a.div.tile.d;   // (n_pairs / 8) * G
        int local = (int)blockIdx.x >> 3;
        if (local >= per_qt * a.n_qtiles) return;
        if (a.perm_n) local = a.perm[local];
        const int jt = udiv(local, a.div.tile);
        qt = a.n_qtiles - 1 - jt;
        const int rem = local - jt * per_qt;
        const int sl = udiv(rem, a.div.g);
        const int p = xcd + 8 * sl;
        b = udiv(p, a.div.hkv);
        h = (p - b * Hkv) * G + (rem - sl * G);
    } else {
        const int bh_count = a.B * Hq;
        const int jt = udiv((int)blockIdx.x, a.div.bhq);
        qt = a.n_qtiles - 1 - jt;
        const int bh = (int)blockIdx.x - jt * bh_count;
        b = udiv(bh, a.div.hq);
        h = bh - b * Hq;
    }
    const int g = udiv(h, a.div.g);

    const int tid = threadIdx.x;
    // The wave index is uniform; readfirstlane lets the compiler keep everything derived
    // from it (the wave's key range, its loop bounds) in scalar registers and branches.
    const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n = lane & 31, hl = lane >> 5;
    const int q0 = qt * C::kBM;
    const int qw = q0 + C::kWQ * wave;   // first query of this wave
    const float c = a.scale_log2;

    const size_t q_stride = (size_t)a.q_rs;     // elements between consecutive t
    const unsigned kv_row_bytes = (unsigned)a.kv_rs * 2u;
    const uint16_t* qbase = a.q + (size_t)b * T * a.q_rs + (size_t)h * D;
    const char* kbase = reinterpret_cast<const char*>(a.k + (size_t)b * T * a.kv_rs + (size_t)g * D);
    const char* vbase = reinterpret_cast<const char*>(a.v + (size_t)b * T * a.kv_rs + (size_t)g * D);

    // Keys needed: up to the last query of the workgroup, with T rounded up to whole
    // waves so that a wave's last block is always loaded (keys past T are masked for
    // every real query).
    const int t_pad = (T + C::kWQ - 1) / C::kWQ * C::kWQ;
    const int kv_end = min(t_pad, q0 + C::kBM);
    const int ntiles = (kv_end + C::kBN - 1) / C::kBN;
    const int nb_wg = (kv_end + 31) / 32;              // 32-key blocks of the workgroup
    const bool active = qw < T;
    const int jd = qw / 32;                            // diagonal block of query block 0
    const int jlast = active ? jd + NQB - 1 : -1;      // the wave's last key block

    // Tile loader: wave instruction i of this wave fills rows
    // kRowsPerLoad * (wave * kLoadsPerTensor + i) + lane / (kRow/16) of the tile, slot
    // lane % (kRow/16), with the logical chunk that the swizzle puts there. Rows past
    // T read row T-1 (finite data; those keys are masked for every real query).
    const int ld_slot = lane % (C::kRow / 16);
    int ld_row[C::kLoadsPerTensor];
    unsigned ld_off[C::kLoadsPerTensor], ld_chunk_b[C::kLoadsPerTensor];
#pragma unroll
    for (int i = 0; i < C::kLoadsPerTensor; ++i) {
        ld_row[i] = C::kRowsPerLoad * (wave * C::kLoadsPerTensor + i) + lane / (C::kRow / 16);
        ld_chunk_b[i] = (unsigned)((ld_slot ^ chunk_swizzle<D>(ld_row[i])) * 16);
        ld_off[i] = (unsigned)ld_row[i] * kv_row_bytes + ld_chunk_b[i];
    }
    auto issue_tile = [&](int jt) CGQA_INLINE {
        char* ks = smem + (jt % C::kStages) * C::kStage;
        char* vs = ks + C::kTile;
        const int row0 = jt * C::kBN;
        const size_t tbase = (size_t)row0 * kv_row_bytes;
#pragma unroll
        for (int i = 0; i < C::kLoadsPerTensor; ++i) {
            const int dst = (wave * C::kLoadsPerTensor + i) * 1024;
            if (row0 + C::kBN <= T) {
                load_lds16_off(kbase + tbase, ld_off[i], ks + dst);
                load_lds16_off(vbase + tbase, ld_off[i], vs + dst);
            } else {
                const unsigned off = (unsigned)min(row0 + ld_row[i], T - 1) * kv_row_bytes + ld_chunk_b[i];
                load_lds16_off(kbase, off, ks + dst);
                load_lds16_off(vbase, off, vs + dst);
            }
        }
    };
    // ROPE: the rotary tables of the K chunks this thread loads (pairs 4c .. 4c+3 of its
    // chunk c, row clamped like the chunk's), by DMA into the thread's own 16 bytes of the
    // cosine and sine areas; after this thread's loads of a tile have landed it turns its
    // own chunks in place (no other thread's data is involved, so only the barrier that
    // publishes the tile follows).
    char* const tab = smem + C::kRing;
    unsigned tab_off[C::kLoadsPerTensor];
#pragma unroll
    for (int i = 0; i < C::kLoadsPerTensor; ++i)
        tab_off[i] = (unsigned)(ld_row[i] * (D / 2) + 4 * (int)(ld_chunk_b[i] / 16)) * 4u;
    auto issue_tables = [&](int jt) CGQA_INLINE {
        const int row0 = jt * C::kBN;
#pragma unroll
        for (int i = 0; i < C::kLoadsPerTensor; ++i) {
            char* dst = tab + (wave * C::kLoadsPerTensor + i) * 1024;
            if (row0 + C::kBN <= T) {
                load_lds16_off(a.rope_cos + (size_t)row0 * (D / 2), tab_off[i], dst);
                load_lds16_off(a.rope_sin + (size_t)row0 * (D / 2), tab_off[i], dst + C::kTabHalf);
            } else {
                const unsigned off = (unsigned)(min(row0 + ld_row[i], T - 1) * (D / 2) + 4 * (int)(ld_chunk_b[i] / 16)) * 4u;
                load_lds16_off(a.rope_cos, off, dst);
                load_lds16_off(a.rope_sin, off, dst + C::kTabHalf);
            }
        }
    };
    auto turn_tile = [&](int jt) CGQA_INLINE {
        char* ks = smem + (jt % C::kStages) * C::kStage;
#pragma unroll
        for (int i = 0; i < C::kLoadsPerTensor; ++i) {
            const int o = (wave * C::kLoadsPerTensor + i) * 1024 + 16 * lane;
            const u32x4 x = *reinterpret_cast<const u32x4*>(ks + o);
            const f32x4 cs = *reinterpret_cast<const f32x4*>(tab + o);
            const f32x4 sn = *reinterpret_cast<const f32x4*>(tab + C::kTabHalf + o);
            *reinterpret_cast<u32x4*>(ks + o) = rope_turn8(x, cs, sn);
        }
    };
    // ROPE, tile t: its loads and its tables were issued before the newest load in
    // flight (tile t + kAhead - 1, issued after the tables of tile t), so waiting for
    // all but that one completes them; turn it, publish it, then load the next tables
    // (this thread's reads of the area are done) and the tile kAhead ahead.
    auto turn_and_advance = [&](int t) CGQA_INLINE {
        static_assert(!ROPE || C::kAhead >= 2, "the wait below assumes a later tile in flight");
        if (t + C::kAhead - 1 < ntiles) wait_vm<C::kLoadsPerTile>();
        else wait_vm<0>();
        turn_tile(t);
        lds_barrier();
        if (t + 1 < ntiles) issue_tables(t + 1);
        if (t + C::kAhead < ntiles) issue_tile(t + C::kAhead);
    };
    // Waits until tile t is in LDS for every wave. Tiles t+1 .. min(t+ahead, ntiles-1)
    // may still be in flight (issued after t, so counted after it).
    auto wait_tile = [&](int t, int ahead) CGQA_INLINE {
        const int later = min(ahead, ntiles - 1 - t);
        if (later >= 2) wait_tiles_barrier<2 * C::kLoadsPerTile>();
        else if (later == 1) wait_tiles_barrier<C::kLoadsPerTile>();
        else wait_tiles_barrier<0>();
    };
    // Loop head of block step j: the step that computes the scores of the first block of
    // tile t = (j + 1) / kBPT waits for that tile and refills the stage of the oldest
    // tile, which no wave reads any more.
    auto head = [&](int j) CGQA_INLINE {
        if ((j + 1) % C::kBPT != 0) return;
        const int t = (j + 1) / C::kBPT;
        if (t >= ntiles) return;
        if constexpr (ROPE) {
            turn_and_advance(t);
        } else {
            wait_tile(t, C::kAhead - 1);
            if (t + C::kAhead < ntiles) issue_tile(t + C::kAhead);
        }
    };

    if constexpr (ROPE) {
        // Tables and tile 0, then tiles 1 .. kAhead-1; the first turn issues the rest.
        if (ntiles > 0) {
            issue_tables(0);
            issue_tile(0);
        }
#pragma unroll
        for (int t = 1; t < C::kAhead; ++t)
            if (t < ntiles) issue_tile(t);
    } else {
#pragma unroll
        for (int t = 0; t <= C::kAhead; ++t)
            if (t < ntiles) issue_tile(t);
    }

    // Q as the B operand: lane (query n of block qb, group hl) holds dims
    // 16*kd + 8*hl .. +7.
    bf16x8 qreg[NQB][C::kKD];
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
        const int row = qw + 32 * qb + n;
#pragma unroll
        for (int kd = 0; kd < C::kKD; ++kd) {
            u32x4 x = {0u, 0u, 0u, 0u};
            if (row < T) {
                x = load16(qbase + (size_t)row * q_stride + 16 * kd + 8 * hl);
                if constexpr (ROPE) {
                    const size_t ti = (size_t)row * (D / 2) + 8 * kd + 4 * hl;
                    x = rope_turn8(x, *reinterpret_cast<const f32x4*>(a.rope_cos + ti),
                                   *reinterpret_cast<const f32x4*>(a.rope_sin + ti));
                }
            }
            qreg[qb][kd] = __builtin_bit_cast(bf16x8, x);
        }
    }
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
        for (int kd = 0; kd < C::kKD; ++kd) asm volatile("" ::"v"(qreg[qb][kd]));

    // Per-lane LDS offsets. K operand: row 32kb + n, logical chunk 2kd + hl. V operand
    // (transposing read): lane j of its 16-lane group reads row 4*hl + j/4 (+8 for the
    // second half) of a 16-row group, 8 bytes at logical column
    // 32mb + 16*((lane>>4)&1) + 4*(j%4). Rows only enter the swizzle through r % 16,
    // which does not depend on the block, so these are per-lane constants; a block adds
    // its stage and row offset as an immediate.
    const char* kaddr[C::kKD];
    const char* vaddr[C::kMB][2];
    {
        const int k_swz = chunk_swizzle<D>(n);
#pragma unroll
        for (int kd = 0; kd < C::kKD; ++kd) kaddr[kd] = smem + n * C::kRow + (((2 * kd + hl) ^ k_swz) << 4);
        const int v_r0 = 4 * hl + ((lane & 15) >> 2);
        const int v_swz[2] = {chunk_swizzle<D>(v_r0), chunk_swizzle<D>(v_r0 + 8)};
        const int v_chunk = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
        const int v_byte = 8 * (lane & 1);
#pragma unroll
        for (int mb = 0; mb < C::kMB; ++mb)
#pragma unroll
            for (int r = 0; r < 2; ++r)
                vaddr[mb][r] = smem + C::kTile + (v_r0 + 8 * r) * C::kRow + v_byte + (((4 * mb + v_chunk) ^ v_swz[r]) << 4);
    }
    // Byte offset of block j's rows (K; V adds kTile through vaddr).
    auto block_off = [](int j) CGQA_INLINE { return ((j / C::kBPT) % C::kStages) * C::kStage + (j % C::kBPT) * 32 * C::kRow; };

    f32x16 oacc[NQB][C::kMB];
    float mref[NQB], lsum[NQB];
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
        mref[qb] = 0.0f;
        lsum[qb] = 0.0f;
#pragma unroll
        for (int mb = 0; mb < C::kMB; ++mb) oacc[qb][mb] = zero16();
    }

    // ---- building blocks of a step. `sel` is a bit set of query blocks.
    auto scores = [&](int boff, int sel, f32x16 (&s)[NQB]) CGQA_INLINE {
        bf16x8 kf[C::kKD];
#pragma unroll
        for (int kd = 0; kd < C::kKD; ++kd) kf[kd] = lds_read8(kaddr[kd] + boff);
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb)
            if (sel >> qb & 1) s[qb] = mfma32x32x16(kf[0], qreg[qb][0], zero16());
#pragma unroll
        for (int kd = 1; kd < C::kKD; ++kd)
#pragma unroll
            for (int qb = 0; qb < NQB; ++qb)
                if (sel >> qb & 1) s[qb] = mfma32x32x16(kf[kd], qreg[qb][kd], s[qb]);
    };
    // O^T += V^T P^T, 16 keys per instruction. B = P straight from the score registers:
    // registers 8t..8t+7 hold keys 16t + 8*(s/4) + 4*hl + s%4 for slot s. A = the same
    // keys of V, read transposed: slots 0..3 from rows 16t + 4*hl + r, slots 4..7 from
    // rows 16t + 8 + 4*hl + r.
    auto pv = [&](int boff, int sel, const bf16x8 (&pb)[NQB][2]) CGQA_INLINE {
        bf16x8 vf[2][C::kMB];
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int mb = 0; mb < C::kMB; ++mb)
                vf[t][mb] = concat(lds_read_tr4(vaddr[mb][0] + boff + 16 * t * C::kRow),
                                   lds_read_tr4(vaddr[mb][1] + boff + 16 * t * C::kRow));
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int mb = 0; mb < C::kMB; ++mb)
#pragma unroll
                for (int qb = 0; qb < NQB; ++qb)
                    if (sel >> qb & 1) oacc[qb][mb] = mfma32x32x16(vf[t][mb], pb[qb][t], oacc[qb][mb]);
    };
    // Diagonal block of query block qb (key block jd + qb): register i is key
    // qw + 32qb + 8(i/4) + 4hl + i%4 against query qw + 32qb + n.
    auto mask_diag = [&](f32x16& s) CGQA_INLINE {
        const int rel = 4 * hl - n;
#pragma unroll
        for (int i = 0; i < 16; ++i)
            if (rel + 8 * (i >> 2) + (i & 3) > 0) s[i] = -INFINITY;
    };
    auto row_max = [&](const f32x16& s) CGQA_INLINE {
        float mx = s[0];
#pragma unroll
        for (int i = 1; i < 16; ++i) mx = fmaxf(mx, s[i]);
        return max_halves(mx) * c;
    };
    // p = 2^(s*c - m) in place; returns this lane's sum; P rounded to bf16 for P.V.
    auto softmax = [&](int qb, f32x16& s, bf16x8 (&pb)[2]) CGQA_INLINE {
        const float nm = -mref[qb];
#pragma unroll
        for (int i = 0; i < 16; ++i) s[i] = exp2_fast(fmaf(s[i], c, nm));
        float t0 = s[0], t1 = s[1];
#pragma unroll
        for (int i = 2; i < 16; i += 2) {
            t0 += s[i];
            t1 += s[i + 1];
        }
        pb[0] = pack_lo(s);
        pb[1] = pack_hi(s);
        return t0 + t1;
    };

    f32x16 s_cur[NQB];
    bf16x8 p_prev[NQB][2];

    // One step j: scores of block j+1 for the query blocks in NX, P.V of block j-1 for
    // those in PV, softmax of block j for those in SM (masked for those in DG). The
    // matrix-core work depends on neither softmax, so the two interleave.
    auto step = [&](int koff_next, int voff_prev, int koff_cur, auto PVc, auto SMc, auto DGc, auto NXc) CGQA_INLINE {
        constexpr int PV = decltype(PVc)::value, SM = decltype(SMc)::value;
        constexpr int DG = decltype(DGc)::value, NX = decltype(NXc)::value;
        f32x16 s_nx[NQB];
        bf16x8 p_cur[NQB][2];
        float t[NQB];
        if constexpr (NX != 0) scores(koff_next, NX, s_nx);
        if constexpr (PV != 0) pv(voff_prev, PV, p_prev);
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb) {
            if (!(SM >> qb & 1)) continue;
            if (DG >> qb & 1) mask_diag(s_cur[qb]);
            t[qb] = softmax(qb, s_cur[qb], p_cur[qb]);
        }
        // Code-generation workaround, measured: this empty unrolled loop keeps the
        // compiler from merging the products and the softmax with the rare-path check
        // below; without it the step takes 12 more registers, 40 more copies and ~10%
        // longer. (An asm statement or sched_barrier here does not have the effect.)
#pragma unroll
        for (int i = 0; i < 8; ++i) {
        }
        bool big = false;
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb)
            if (SM >> qb & 1) big |= !(t[qb] <= kRescaleLimit);
        if (wave_any(big)) {
            // Rare: some score rose far above the reference. Recompute the block's
            // scores, move the reference to the row max and rescale what was summed so
            // far.
            f32x16 s2[NQB];
            scores(koff_cur, SM, s2);
#pragma unroll
            for (int qb = 0; qb < NQB; ++qb) {
                if (!(SM >> qb & 1)) continue;
                if (DG >> qb & 1) mask_diag(s2[qb]);
                const float mnew = fmaxf(mref[qb], row_max(s2[qb]));
                const float alpha = exp2_fast(mref[qb] - mnew);
                mref[qb] = mnew;
                lsum[qb] *= alpha;
#pragma unroll
                for (int mb = 0; mb < C::kMB; ++mb)
#pragma unroll
                    for (int i = 0; i < 16; ++i) oacc[qb][mb][i] *= alpha;
                s_cur[qb] = s2[qb];
                t[qb] = softmax(qb, s_cur[qb], p_cur[qb]);
            }
        }
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb) {
            if (SM >> qb & 1) {
                lsum[qb] += t[qb];
                p_prev[qb][0] = p_cur[qb][0];
                p_prev[qb][1] = p_cur[qb][1];
            }
            if (NX >> qb & 1) s_cur[qb] = s_nx[qb];
        }
    };
    using I0 = std::integral_constant<int, 0>;
    using IAll = std::integral_constant<int, kAll>;

        // the matrix core beside the softmax of block j.
        // ---- prologue: tile 0, scores of block 0 and the reference maximum.
        if constexpr (ROPE) {
            if (ntiles > 0) turn_and_advance(0);
        } else {
            wait_tile(0, C::kAhead);
        }
        if (active) {
            scores(0, kAll, s_cur);
            f32x16 sm = s_cur[0];
            if (jd == 0) mask_diag(sm);
            mref[0] = row_max(sm);
        }
        if (active && jd >= 1) {
            // Step 0: no P.V yet.
            head(0);
            step(block_off(1), 0, block_off(0), I0{}, IAll{}, I0{}, IAll{});
            // Steady steps 1 .. jd-1, unrolled by the period of the stage map so that
            // every LDS address is a per-lane register plus an immediate.
            for (int j0 = 0; j0 < jd; j0 += C::kUnroll) {
                static_for<C::kUnroll>([&](auto Uc) CGQA_INLINE {
                    constexpr int U = decltype(Uc)::value;
                    const int j = j0 + U;
                    if (j == 0 || j >= jd) return;
                    if constexpr ((U + 1) % C::kBPT == 0) head(j);
                    constexpr int off_next = block_off((U + 1) % C::kUnroll);
                    constexpr int off_cur = block_off(U);
                    constexpr int off_prev = block_off((U + C::kUnroll - 1) % C::kUnroll);
                    step(off_next, off_prev, off_cur, IAll{}, IAll{}, I0{}, IAll{});
                });
            }
        }
        if (active) {
            // Step jd: the diagonal block, then its own P.V.
            head(jd);
            if (jd >= 1)
                step(0, block_off(jd - 1), block_off(jd), IAll{}, IAll{}, IAll{}, I0{});
            else
                step(0, 0, block_off(jd), I0{}, IAll{}, IAll{}, I0{});
            pv(block_off(jd), kAll, p_prev);
        }
    // Steps after this wave's last block: keep the workgroup's barriers and loads going.
    for (int j = jlast + 1; j < nb_wg; ++j) head(j);

    // ---- epilogue: O = acc / l in bf16, LSE = ln2 * (m + log2 l).
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
        const int query = qw + 32 * qb + n;
        if (!active || query >= T) continue;
        const float l = sum_halves(lsum[qb]);
        const float inv = 1.0f / l;
        uint16_t* orow = a.o + ((size_t)b * T + query) * a.o_rs + (size_t)h * D;
#pragma unroll
        for (int mb = 0; mb < C::kMB; ++mb) {
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                f32x4 x;
#pragma unroll
                for (int r = 0; r < 4; ++r) x[r] = oacc[qb][mb][4 * u + r] * inv;
                const bf16x4 y = __builtin_convertvector(x, bf16x4);
                *reinterpret_cast<u32x2*>(orow + 32 * mb + 8 * u + 4 * hl) = __builtin_bit_cast(u32x2, y);
            }
        }
        if (hl == 0) a.lse[((size_t)b * Hq + h) * T + query] = (mref[qb] + log2_fast(l)) * kLn2;
    }
}

template <int D, bool ROPE>
static hipError_t launch_fwd_t(const FwdArgs& a, hipStream_t stream) {
    using C = FwdCfg<D, ROPE>;
    FwdArgs x = a;
    x.n_qtiles = (a.T + C::kBM - 1) / C::kBM;
    x.n_pairs = a.B * a.Hkv;
    x.xcd_group = x.n_pairs % 8 == 0 ? 1 : 0;
    x.perm_n = 0;
    if (x.xcd_group) {
        // Work of a query tile: the key blocks of its waves (a wave's prologue and
        // epilogue count about two more).
        const int per_qt = a.div.tile.d, nqt = x.n_qtiles, T = a.T;
        auto weight = [&](int p) {
            const int qt = nqt - 1 - p / per_qt;
            long w = 0;
            for (int wv = 0; wv < C::kWaves; ++wv) {
                const int qw = qt * C::kBM + C::kWQ * wv;
                if (qw < T) w += qw / 32 + 1 + 2;
            }
            return w;
        };
        x.perm_n = balance_one_round(x.perm, per_qt * nqt, cus_per_xcd(), C::kResident, weight);
    }
    const long blocks = (long)x.n_qtiles * a.B * a.Hq;
    hipLaunchKernelGGL((attn_fwd_kernel<D, ROPE>), dim3((unsigned)blocks), dim3(C::kThreads), 0, stream, x);
    return hipGetLastError();
}

// Forward kernel choice, by shape alone: d = 64 grids too small to fill the chip go to the
// key-split kernel (attn_fwd_par.hip), every other shape to the tiled kernel above.
hipError_t launch_fwd(const FwdArgs& a, hipStream_t stream) {
    if (fwd_split_keys_chosen(a)) return launch_fwd_split_keys(a, stream);
    if (a.d == 64) return launch_fwd_t<64, false>(a, stream);
    return launch_fwd_t<128, false>(a, stream);
}

// The rotary forward (d = 64) always runs the tiled kernel (the key-split one has no
// rotary variant).
hipError_t launch_fwd_rope(const FwdArgs& a, hipStream_t stream) {
    if (a.d != 64) return hipErrorInvalidValue;
    return launch_fwd_t<64, true>(a, stream);
}

}  // namespace cgqa
