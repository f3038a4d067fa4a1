// Forward kernel of causal grouped-query flash attention for gfx950, balanced variant
// for head dimension 64, three query heads per kv head and sequence lengths that are a
// multiple of 64.
//
// The method is the one of attn_fwd.hip (page "A transformer in PTX", section "Flash
// attention": online softmax in base-2 units over key blocks up to the diagonal, O =
// acc / l, the natural-log LSE stored for the backward). What differs is how the causal
// triangle is cut into work and how K and V reach LDS.
//
// Under the causal mask the last block of queries needs every key block, so when one
// wave owns a query block from its first key to its last, the wave with the last block
// alone sets the kernel's length, however many CUs are idle. Here a workgroup takes a
// (batch, kv head) slice and the pair of 64-query blocks i and j = n-1-i (n = T / 64).
// Together they need 2n + 2 steps of 32 keys; two waves per query head share them
// evenly:
//   wave A: all of block i (keys 0 .. 64i+63), then keys 0 .. 32(n-1-2i)-1 of block j;
//   wave B: the remaining keys of block j, up to its diagonal.
// Each has n + 1 steps. Softmax lets the two partial results of block j (reference max,
// sum and unnormalised output of each wave) be merged exactly through LDS at the end.
// With n odd the middle block pairs with itself and wave A alone takes it.
//
// Every wave streams its own K and V blocks from global memory into a private ring of
// three LDS stages by DMA and waits only for its own loads: no workgroup barrier until
// the final merge. (On gfx950 a barrier per step holds the waves in lockstep and costs
// more than the extra L2 traffic of unshared streams; the three heads of a group still
// share K and V through the L2 of their XCD.) Wave A's ring also carries block j's Q,
// loaded one slot before the wave moves on to block j.
//
// Inside a wave the step is the same two-phase ping-pong as in attn_fwd.hip: phase 1
// runs the scores of query half 1 and its P.V product on the matrix core beside the
// softmax of query half 0; phase 2 runs half 0's P.V product and next scores beside
// half 1's softmax.
#include "cgqa_device.hpp"
#include "cgqa_launch.hpp"

#include <type_traits>

namespace cgqa {

struct SplitCfg {
    static constexpr int D = 64;
    static constexpr int kG = 3;                            // query heads per kv head
    static constexpr int kWaves = 2 * kG;
    static constexpr int kKD = D / 16;                      // k-steps over the head dimension
    static constexpr int kMB = D / 32;                      // 32-dim blocks of the output
    static constexpr int kRow = D * 2;                      // bytes per K or V row in LDS
    static constexpr int kBlk = 32 * kRow;                  // K (or V) of one 32-key block
    static constexpr int kStage = 2 * kBlk;                 // one ring slot: K then V, or a Q block
    static constexpr int kStages = 3;
    static constexpr int kRing = kStages * kStage;          // one wave's ring
    static constexpr int kLds = kWaves * kRing;
    static constexpr int kLoads = 8;                        // 1 KB DMA instructions per slot
    // Partial result of one head for the merge, in accumulator-register order: O (two
    // query halves x kMB blocks x 16 registers x 64 lanes), then m and l (2 x 64 each).
    static constexpr int kPartO = 2 * kMB * 16 * 64 * 4;
    static constexpr int kPart = kPartO + 2 * 2 * 64 * 4;
    static_assert(kG * kPart <= kLds, "merge area reuses the rings");
    static_assert(kLds <= 160 * 1024, "LDS budget");
    static_assert(kStage == 64 * kRow, "a Q block fills one slot");
};

// Probabilities above this trigger a move of the reference max.
constexpr float kSplitRescaleLimit = 1099511627776.0f;   // 2^40

__global__ __launch_bounds__(SplitCfg::kWaves * 64, 1) void attn_fwd_split_kernel(FwdArgs a) {
    using C = SplitCfg;
    constexpr int D = C::D;
    constexpr int S = C::kStages;
    __shared__ __attribute__((aligned(1024))) char smem[C::kLds];

    const int T = a.T, Hq = a.Hq, Hkv = a.Hkv;
    constexpr int G = C::kG;
    const int P = a.n_pairs;                 // B * Hkv slices
    const int nq = T / 64;                   // 64-query blocks per head
    const int pair = (int)blockIdx.x / P, slice = (int)blockIdx.x % P;
    const int b = slice / Hkv, g = slice % Hkv;
    const int iq = pair, jq = nq - 1 - pair;
    const bool middle = iq == jq;
    const int nsteps = nq + 1;

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n = lane & 31, hl = lane >> 5;
    const int half = wave / G;               // 0: wave A, 1: wave B
    const int hg = wave - half * G;          // head within the group
    const int h = g * G + hg;
    const float c = a.scale_log2;
    const bool active = !(middle && half == 1);
    const bool switches = half == 0 && !middle;   // wave A with a part of block j

    const size_t q_stride = (size_t)Hq * D;
    const unsigned kv_row_bytes = (unsigned)(Hkv * D * 2);
    const unsigned q_row_bytes = (unsigned)(Hq * D * 2);
    const uint16_t* qbase = a.q + ((size_t)b * T * Hq + h) * D;
    const char* kbase = reinterpret_cast<const char*>(a.k + ((size_t)b * T * Hkv + g) * D);
    const char* vbase = reinterpret_cast<const char*>(a.v + ((size_t)b * T * Hkv + g) * D);
    char* ring = smem + wave * C::kRing;

    // ---- the wave's slots. Wave A (switching): K/V of block i's key blocks 0..2i+1,
    // then block j's Q, then K/V of block j's key blocks 0..n-2-2i. Wave A of the middle
    // block: its key blocks 0..n. Wave B: key blocks n-1-2i .. 2n-1-2i of block j.
    // Step s reads slot x(s) = s, or s + 1 after wave A's switch.
    const int q_slot = switches ? 2 * iq + 2 : -1;
    const int n_slots = !active ? 0 : switches ? nq + 2 : nq + 1;
    auto slot_of = [&](int s) CGQA_INLINE { return (switches && s >= 2 * iq + 2) ? s + 1 : s; };
    unsigned kv_off[4], q_off[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        // K or V rows 8e .. 8e+7: lane -> row 8e + lane/8, 16-byte slot lane % 8 holding
        // the logical chunk that the swizzle puts there.
        const int r = 8 * e + (lane >> 3);
        kv_off[e] = (unsigned)r * kv_row_bytes + (unsigned)(((lane & 7) ^ chunk_swizzle<D>(r)) * 16);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        // Q register group e = qb * kKD + kd, in register order (lane -> 16 bytes).
        const int qb = e / C::kKD, kd = e % C::kKD;
        q_off[e] = (unsigned)(64 * jq + 32 * qb + n) * q_row_bytes + (unsigned)((16 * kd + 8 * hl) * 2);
    }
    int issued_hi = -1;   // highest slot issued so far
    auto issue = [&](int x) CGQA_INLINE {
        if (x >= n_slots) return;
        issued_hi = x;   // slots are issued in order
        char* dst = ring + (x % S) * C::kStage;
        if (x == q_slot) {
            const char* src = reinterpret_cast<const char*>(qbase);
#pragma unroll
            for (int e = 0; e < 8; ++e) load_lds16_off(src, q_off[e], dst + 1024 * e);
            return;
        }
        const int kb = half == 1 ? nq - 1 - 2 * iq + x : (switches && x > q_slot) ? x - q_slot - 1 : x;
        const size_t row0 = (size_t)(32 * kb) * kv_row_bytes;
#pragma unroll
        for (int e = 0; e < 4; ++e) load_lds16_off(kbase + row0, kv_off[e], dst + 1024 * e);
#pragma unroll
        for (int e = 0; e < 4; ++e) load_lds16_off(vbase + row0, kv_off[e], dst + C::kBlk + 1024 * e);
    };
    // Wait until slot x is in LDS (slots issued after it may stay in flight).
    auto wait_slot = [&](int x) CGQA_INLINE {
        const int later = issued_hi - x;
        if (later >= 2) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * C::kLoads) : "memory");
        else if (later == 1) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(C::kLoads) : "memory");
        else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    };
    // Issue the slots after the last one issued, up to slot y. A slot may be issued once
    // the slot three before it (same stage) has been read for the last time.
    auto issue_upto = [&](int y) CGQA_INLINE {
#pragma unroll
        for (int i = 0; i < S; ++i)
            if (issued_hi < y) issue(issued_hi + 1);
    };
    // Head of step s: every slot before x(s) has been consumed (its K and V are in
    // registers or used), so slots up to x(s) + 2 may be issued; with `next`, wait for
    // the next step's slot, whose K this step reads early.
    auto head = [&](int s, bool next) CGQA_INLINE {
        issue_upto(slot_of(s) + 2);
        if (next) wait_slot(slot_of(s + 1));
    };
    issue(0);
    issue(1);

    // ---- Q of the wave's first query block as the B operand: lane (query n of half
    // qb, group hl) holds dims 16*kd + 8*hl .. +7.
    bf16x8 qreg[2][C::kKD];
    {
        const int qblk = half == 0 ? iq : jq;
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
#pragma unroll
            for (int kd = 0; kd < C::kKD; ++kd)
                qreg[qb][kd] = __builtin_bit_cast(
                    bf16x8, load16(qbase + (size_t)(64 * qblk + 32 * qb + n) * q_stride + 16 * kd + 8 * hl));
    }

    // Per-lane LDS addresses in this wave's ring. K operand: row n, logical chunk
    // 2kd + hl. V operand (transposing read): lane j of a 16-lane group reads row
    // 4*hl + j/4 (+8 for the second half) of a 16-row group, 8 bytes at logical column
    // 32mb + 16*((lane>>4)&1) + 4*(j%4).
    const char* kaddr[C::kKD];
    const char* vaddr[C::kMB][2];
    {
        const int k_swz = chunk_swizzle<D>(n);
#pragma unroll
        for (int kd = 0; kd < C::kKD; ++kd) kaddr[kd] = ring + n * C::kRow + (((2 * kd + hl) ^ k_swz) << 4);
        const int v_r0 = 4 * hl + ((lane & 15) >> 2);
        const int v_swz[2] = {chunk_swizzle<D>(v_r0), chunk_swizzle<D>(v_r0 + 8)};
        const int v_chunk = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
        const int v_byte = 8 * (lane & 1);
#pragma unroll
        for (int mb = 0; mb < C::kMB; ++mb)
#pragma unroll
            for (int r = 0; r < 2; ++r)
                vaddr[mb][r] = ring + C::kBlk + (v_r0 + 8 * r) * C::kRow + v_byte + (((4 * mb + v_chunk) ^ v_swz[r]) << 4);
    }

    f32x16 oacc[2][C::kMB];
    float mref[2], lsum[2];
    auto reset = [&]() CGQA_INLINE {
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
            mref[qb] = 0.0f;
            lsum[qb] = 0.0f;
#pragma unroll
            for (int mb = 0; mb < C::kMB; ++mb) oacc[qb][mb] = zero16();
        }
    };
    reset();
    f32x16 s_cur[2];
    bf16x8 p_prev[2][2];
    bf16x8 kf[C::kKD], vf[2][C::kMB];

    auto read_kf = [&](int boff) CGQA_INLINE {
#pragma unroll
        for (int kd = 0; kd < C::kKD; ++kd) kf[kd] = lds_read8(kaddr[kd] + boff);
    };
    auto read_vf = [&](int boff) CGQA_INLINE {
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int mb = 0; mb < C::kMB; ++mb)
                vf[t][mb] = concat(lds_read_tr4(vaddr[mb][0] + boff + 16 * t * C::kRow),
                                   lds_read_tr4(vaddr[mb][1] + boff + 16 * t * C::kRow));
    };
    // S^T = K Q^T for query half qb (rows: keys, columns: queries).
    auto s_mfma = [&](int qb, const bf16x8 (&k)[C::kKD], f32x16& sc) CGQA_INLINE {
        sc = mfma32x32x16(k[0], qreg[qb][0], zero16());
#pragma unroll
        for (int kd = 1; kd < C::kKD; ++kd) sc = mfma32x32x16(k[kd], qreg[qb][kd], sc);
    };
    // O^T += V^T P^T with P straight from the score registers (registers 8t..8t+7 hold
    // keys 16t + 8*(s/4) + 4*hl + s%4 for slot s; V read transposed to match).
    auto pv_mfma = [&](int qb, const bf16x8 (&pb)[2]) CGQA_INLINE {
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int mb = 0; mb < C::kMB; ++mb) oacc[qb][mb] = mfma32x32x16(vf[t][mb], pb[t], oacc[qb][mb]);
    };
    // Diagonal block of a query half: register i is key 8(i/4) + 4hl + i%4 of the block
    // against query n of the half.
    auto mask_diag = [&](f32x16& sc) CGQA_INLINE {
        const int rel = 4 * hl - n;
#pragma unroll
        for (int i = 0; i < 16; ++i)
            if (rel + 8 * (i >> 2) + (i & 3) > 0) sc[i] = -INFINITY;
    };
    auto row_max = [&](const f32x16& sc) CGQA_INLINE {
        float mx = sc[0];
#pragma unroll
        for (int i = 1; i < 16; ++i) mx = fmaxf(mx, sc[i]);
        return max_halves(mx) * c;
    };
    // p = 2^(s*c - m) in place; returns this lane's sum; P rounded to bf16 for P.V.
    auto softmax = [&](int qb) CGQA_INLINE {
        f32x16& sc = s_cur[qb];
        const float nm = -mref[qb];
#pragma unroll
        for (int i = 0; i < 16; ++i) sc[i] = exp2_fast(fmaf(sc[i], c, nm));
        float t0 = sc[0], t1 = sc[1];
#pragma unroll
        for (int i = 2; i < 16; i += 2) {
            t0 += sc[i];
            t1 += sc[i + 1];
        }
        p_prev[qb][0] = pack_lo(sc);
        p_prev[qb][1] = pack_hi(sc);
        return t0 + t1;
    };
    // Rare path: some score rose far above the reference. Recompute the block's scores
    // (K fragments `k`), move the reference to the row max and rescale what was summed.
    auto rebase = [&](int qb, const bf16x8 (&k)[C::kKD], bool diag) CGQA_INLINE {
        f32x16 s2;
        s_mfma(qb, k, s2);
        if (diag) mask_diag(s2);
        const float mnew = fmaxf(mref[qb], row_max(s2));
        const float alpha = exp2_fast(mref[qb] - mnew);
        mref[qb] = mnew;
        lsum[qb] *= alpha;
#pragma unroll
        for (int mb = 0; mb < C::kMB; ++mb)
#pragma unroll
            for (int i = 0; i < 16; ++i) oacc[qb][mb][i] *= alpha;
        s_cur[qb] = s2;
        return softmax(qb);
    };
    // Softmax of query half qb at step s with its rare-path check. FROM_KF: kf still
    // holds the block's K; otherwise it is read again from LDS.
    auto finish = [&](int qb, float t, int s_off, bool diag, auto FROM_KF) CGQA_INLINE {
        if (wave_any(!(t <= kSplitRescaleLimit))) {
            if constexpr (decltype(FROM_KF)::value) {
                t = rebase(qb, kf, diag);
            } else {
                bf16x8 k2[C::kKD];
#pragma unroll
                for (int kd = 0; kd < C::kKD; ++kd) k2[kd] = lds_read8(kaddr[kd] + s_off);
                t = rebase(qb, k2, diag);
            }
        }
        lsum[qb] += t;
    };
    using KF = std::true_type;
    using LDSK = std::false_type;
    // Interleave hint for one phase of a steady step (8 matrix-core instructions spread
    // through the softmax); in phase 1 the K reads for the next step follow the scores
    // that used the old fragments and the V reads follow the P.V products.
    auto hint = [&](auto PHASE1) CGQA_INLINE {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            CGQA_SCHED_GROUP(kSchedMFMA, 1);
            CGQA_SCHED_GROUP(kSchedVALU, 8);
        }
        if constexpr (decltype(PHASE1)::value) CGQA_SCHED_GROUP(kSchedDSRead, C::kKD);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            CGQA_SCHED_GROUP(kSchedMFMA, 1);
            CGQA_SCHED_GROUP(kSchedVALU, 8);
        }
        if constexpr (decltype(PHASE1)::value) CGQA_SCHED_GROUP(kSchedDSRead, 4 * C::kMB);
    };
    // Scores of both halves for the first block of a range (slot offset boff), and the
    // reference maxima.
    auto range_prologue = [&](int boff, bool mask0) CGQA_INLINE {
        read_kf(boff);
        s_mfma(0, kf, s_cur[0]);
        s_mfma(1, kf, s_cur[1]);
        f32x16 sm = s_cur[0];
        if (mask0) mask_diag(sm);
        mref[0] = row_max(sm);
        mref[1] = row_max(s_cur[1]);
    };
    // Ring offset of step s's slot; SH = 1 for the steps of wave A after its switch.
    auto soff = [](int s, auto SH) CGQA_INLINE { return ((s + decltype(SH)::value) % S) * C::kStage; };
    // Steady steps s_first .. s_end-1 (each has a next block and a previous P.V),
    // unrolled by the ring length so that every LDS address is a register plus an
    // immediate.
    auto steady = [&](int s_first, int s_end, auto SH) CGQA_INLINE {
        constexpr int sh = decltype(SH)::value;
        for (int s_base = s_first - s_first % S; s_base < s_end; s_base += S) {
            static_for<S>([&](auto Uc) CGQA_INLINE {
                constexpr int U = decltype(Uc)::value;
                const int s = s_base + U;
                if (s < s_first || s >= s_end) return;
                head(s, true);
                constexpr int off_cur = ((U + sh) % S) * C::kStage;
                constexpr int off_next = ((U + sh + 1) % S) * C::kStage;
                // phase 1
                s_mfma(1, kf, s_cur[1]);
                pv_mfma(1, p_prev[1]);
                read_kf(off_next);
                read_vf(off_cur);
                const float ta = softmax(0);
                hint(std::true_type{});
                finish(0, ta, off_cur, false, LDSK{});
                // phase 2
                pv_mfma(0, p_prev[0]);
                s_mfma(0, kf, s_cur[0]);
                const float tb = softmax(1);
                hint(std::false_type{});
                finish(1, tb, off_cur, false, LDSK{});
            });
        }
    };
    // First step of a range (no P.V yet); `more`: the range has a next block.
    auto first_step = [&](int s0, bool more, auto SH) CGQA_INLINE {
        head(s0, more);
        finish(0, softmax(0), soff(s0, SH), false, KF{});
        if (more) read_kf(soff(s0 + 1, SH));
        read_vf(soff(s0, SH));
        pv_mfma(0, p_prev[0]);
        if (more) s_mfma(0, kf, s_cur[0]);
        finish(1, softmax(1), soff(s0, SH), false, LDSK{});
    };
    // A range of L >= 2 steps from s0 that ends at the diagonals of both query halves
    // (half 0 at step s0+L-2, half 1 at s0+L-1).
    auto run_diag = [&](int s0, int L) CGQA_INLINE {
        using SH = std::integral_constant<int, 0>;
        const int jd = s0 + L - 2;
        wait_slot(slot_of(s0));
        range_prologue(soff(s0, SH{}), L == 2);
        if (L >= 3) {
            first_step(s0, true, SH{});
            steady(s0 + 1, jd, SH{});
        }
        // step jd: diagonal of half 0
        head(jd, true);
        if (L >= 3) {
            s_mfma(1, kf, s_cur[1]);
            pv_mfma(1, p_prev[1]);
        }
        mask_diag(s_cur[0]);
        finish(0, softmax(0), soff(jd, SH{}), true, KF{});
        read_vf(soff(jd, SH{}));
        pv_mfma(0, p_prev[0]);
        finish(1, softmax(1), soff(jd, SH{}), false, LDSK{});
        // step jd+1: diagonal of half 1
        head(jd + 1, false);
        read_kf(soff(jd + 1, SH{}));
        s_mfma(1, kf, s_cur[1]);
        pv_mfma(1, p_prev[1]);
        mask_diag(s_cur[1]);
        finish(1, softmax(1), soff(jd + 1, SH{}), true, KF{});
        read_vf(soff(jd + 1, SH{}));
        pv_mfma(1, p_prev[1]);
    };
    // Wave A's part of block j: L >= 1 steps from s0, strictly below both diagonals.
    auto run_plain = [&](int s0, int L) CGQA_INLINE {
        using SH = std::integral_constant<int, 1>;
        wait_slot(slot_of(s0));
        range_prologue(soff(s0, SH{}), false);
        first_step(s0, L >= 2, SH{});
        if (L >= 2) {
            const int sl = s0 + L - 1;
            steady(s0 + 1, sl, SH{});
            // last step: no next block
            head(sl, false);
            s_mfma(1, kf, s_cur[1]);
            pv_mfma(1, p_prev[1]);
            read_vf(soff(sl, SH{}));
            finish(0, softmax(0), soff(sl, SH{}), false, LDSK{});
            pv_mfma(0, p_prev[0]);
            finish(1, softmax(1), soff(sl, SH{}), false, KF{});
        }
        pv_mfma(1, p_prev[1]);
    };
    // O = acc / l in bf16 and LSE = ln2 * (m + log2 l) for 64-query block qblk.
    auto finalize = [&](int qblk) CGQA_INLINE {
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
            const int query = 64 * qblk + 32 * qb + n;
            const float l = sum_halves(lsum[qb]);
            const float inv = 1.0f / l;
            uint16_t* orow = a.o + ((size_t)b * T + query) * q_stride + (size_t)h * D;
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
    };

    if (switches) {
        run_diag(0, 2 * iq + 2);
        // Block i's last slot is consumed: refill the ring before the stores of block i.
        issue_upto(2 * iq + 4);
        finalize(iq);
        reset();
        // block j's Q from its slot, then block j's keys from 0
        wait_slot(q_slot);
        const char* qs = ring + (q_slot % S) * C::kStage;
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
#pragma unroll
            for (int kd = 0; kd < C::kKD; ++kd)
                qreg[qb][kd] = __builtin_bit_cast(
                    bf16x8, *reinterpret_cast<const u32x4*>(qs + ((qb * C::kKD + kd) * 64 + lane) * 16));
        run_plain(2 * iq + 2, nq - 1 - 2 * iq);
    } else if (active) {
        run_diag(0, nsteps);
        if (middle) finalize(iq);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    if (middle) return;

    // ---- merge the two halves of block j through LDS (the rings are free now)
    wait_tiles_barrier<0>();
    char* part = smem + hg * C::kPart;
    float* part_ml = reinterpret_cast<float*>(part + C::kPartO);
    if (half == 0) {
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
#pragma unroll
            for (int mb = 0; mb < C::kMB; ++mb)
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    f32x4 x;
#pragma unroll
                    for (int r = 0; r < 4; ++r) x[r] = oacc[qb][mb][4 * u + r];
                    *reinterpret_cast<f32x4*>(part + (((qb * C::kMB + mb) * 4 + u) * 64 + lane) * 16) = x;
                }
            part_ml[qb * 64 + lane] = mref[qb];
            part_ml[128 + qb * 64 + lane] = lsum[qb];
        }
    }
    wait_tiles_barrier<0>();
    if (half == 1) {
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
            const float ma = part_ml[qb * 64 + lane];
            const float la = part_ml[128 + qb * 64 + lane];
            const float m = fmaxf(ma, mref[qb]);
            const float aa = exp2_fast(ma - m), ab = exp2_fast(mref[qb] - m);
            lsum[qb] = la * aa + lsum[qb] * ab;
            mref[qb] = m;
#pragma unroll
            for (int mb = 0; mb < C::kMB; ++mb)
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const f32x4 x = *reinterpret_cast<const f32x4*>(part + (((qb * C::kMB + mb) * 4 + u) * 64 + lane) * 16);
#pragma unroll
                    for (int r = 0; r < 4; ++r) oacc[qb][mb][4 * u + r] = x[r] * aa + oacc[qb][mb][4 * u + r] * ab;
                }
        }
        finalize(jq);
    }
}

// Shapes the balanced kernel handles: d = 64, whole 64-query blocks (at least two),
// three query heads per kv head.
// Contiguous tensors only (the kernel derives its row strides from the head counts).
bool fwd_split_supported(const FwdArgs& a) {
    return a.d == 64 && a.T % 64 == 0 && a.T >= 128 && a.Hq == SplitCfg::kG * a.Hkv &&
           a.q_rs == a.Hq * a.d && a.kv_rs == a.Hkv * a.d && a.o_rs == a.Hq * a.d;
}

// Workgroups of the balanced kernel: one per (pair of query blocks, batch, kv head).
long fwd_split_blocks(const FwdArgs& a) { return (long)(a.T / 64 + 1) / 2 * a.B * a.Hkv; }

hipError_t launch_fwd_split(const FwdArgs& a, hipStream_t stream) {
    FwdArgs x = a;
    x.n_pairs = a.B * a.Hkv;
    hipLaunchKernelGGL(attn_fwd_split_kernel, dim3((unsigned)fwd_split_blocks(a)), dim3(SplitCfg::kWaves * 64), 0,
                       stream, x);
    return hipGetLastError();
}

}  // namespace cgqa
