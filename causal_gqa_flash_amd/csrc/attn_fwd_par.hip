// Forward kernel of causal grouped-query flash attention for gfx950, with the key range of
// every query block split in two (even and odd key blocks) and the causal triangle cut
// into many short workgroups.
//
// The method is the one of attn_fwd.hip (page "A transformer in PTX", section "Flash
// attention": online softmax in base-2 units over the key blocks up to the diagonal,
// O = acc / l, the natural-log LSE stored for the backward). What differs is the work
// split. Under the causal mask query block q needs q + 1 key blocks; when one wave owns a
// query block from its first key to its diagonal, the waves with the last blocks set the
// kernel's length while most of the chip idles. Here a workgroup of four waves takes a
// 64-query tile (two 32-query blocks) of one head, and each query block is shared by two
// waves: one takes the even key blocks, the other the odd ones. A tile then needs
// tile + 1 steps instead of 2 (tile + 1), and there are twice as many workgroups as the
// chip holds at once (three per CU), so with the heaviest tiles dispatched first the
// light ones fill the CUs as the heavy ones finish. Softmax lets the two halves of a
// query block (reference max, sum and unnormalised output of each) be merged exactly
// through LDS at the end, in a fixed order.
//
// Step s of a workgroup covers key blocks 2s and 2s+1 (a 64-key stage). K and V go
// straight from global memory to LDS (global_load_lds_dwordx4) into a three-slot ring:
// slot u % 3 holds K of stage u and V of stage u - 1, because a step reads the scores'
// K one stage ahead of the P.V product's V. Each wave copies one 32-key tile per step
// (K or V, even or odd). One barrier per step; the loads of step s + 1's K (and step s's
// V) are issued one step ahead.
//
// Inside a wave a step is the pipelined step of attn_fwd.hip: the scores of the wave's
// next key block and the P.V product of its previous one on the matrix core beside the
// softmax of the current block on the vector ALU, the causal mask only on the diagonal,
// and a lazy reference max. Tiles of one (batch, kv head) slice run on one XCD (as in the
// tiled kernel), whose L2 then serves that slice's K and V to every head of the group.
#include "cgqa_device.hpp"
#include "cgqa_launch.hpp"

#include <type_traits>

namespace cgqa {

template <int D>
struct ParCfg {
    static constexpr int kWaves = 4;
    static constexpr int kThreads = 64 * kWaves;
    static constexpr int kBM = 64;                      // queries per workgroup
    static constexpr int kKD = D / 16;                  // k-steps over the head dimension
    static constexpr int kMB = D / 32;                  // 32-dim blocks of the output
    static constexpr int kRow = D * 2;                  // bytes per K or V row in LDS
    static constexpr int kTile = 32 * kRow;             // K or V of one 32-key block
    static constexpr int kChunks = kTile / 1024;        // 1 KB DMA instructions per tile
    static constexpr int kRowsPerChunk = 1024 / kRow;
    static constexpr int kSlots = 3;
    static constexpr int kSlot = 4 * kTile;             // K even, K odd, V even, V odd
    static constexpr int kLds = kSlots * kSlot;
    // Partial result of one query block for the merge: O accumulators (kMB x 16 per lane),
    // then the reference max and the lane's partial sum.
    static constexpr int kPartO = kMB * 16 * 64 * 4;
    static constexpr int kPart = kPartO + 2 * 64 * 4;
    static_assert(D == 64 || D == 128, "head dim");
    static_assert(2 * kPart <= kLds, "merge area reuses the ring");
    static_assert(kLds <= 160 * 1024, "LDS budget");
};

// Probabilities above this trigger a move of the reference max.
constexpr float kParRescaleLimit = 1099511627776.0f;   // 2^40

template <int D>
__global__ __launch_bounds__(256, D == 64 ? 3 : 2) void attn_fwd_par_kernel(FwdArgs a) {
    using C = ParCfg<D>;
    __shared__ __attribute__((aligned(1024))) char smem[C::kLds];

    const int T = a.T, Hq = a.Hq, Hkv = a.Hkv;
    const int G = a.div.G;
    int qt, b, h;
    if (a.xcd_group) {
        // Slices p = b * Hkv + g with p % 8 == x % 8 run on XCD x % 8 (n_pairs % 8 == 0);
        // on each XCD the heaviest tiles are dispatched first.
        const int xcd = (int)blockIdx.x & 7;
        const int per_qt = a.div.tile.d;   // (n_pairs / 8) * G
        const int local = (int)blockIdx.x >> 3;
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
    const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n = lane & 31, hl = lane >> 5;
    const int par = wave & 1;                           // key blocks of this parity
    const int qb = 2 * qt + (wave >> 1);                // this wave's 32-query block
    const float c = a.scale_log2;
    const int nkb = (T + 31) / 32;
    // Key blocks par, par + 2, ... up to the query block's diagonal: my_len of them, in
    // stages 0 .. my_len - 1. The diagonal one, if this parity has it, is the last.
    const bool valid = 32 * qb < T;
    const int my_len = valid && qb >= par ? (qb - par) / 2 + 1 : 0;
    const bool my_diag = my_len > 0 && 2 * (my_len - 1) + par == qb;
    const int nsteps = qt + 1;                          // stages of the workgroup

    const unsigned kv_row_bytes = (unsigned)a.kv_rs * 2u;
    const char* kbase = reinterpret_cast<const char*>(a.k + (size_t)b * T * a.kv_rs + (size_t)g * D);
    const char* vbase = reinterpret_cast<const char*>(a.v + (size_t)b * T * a.kv_rs + (size_t)g * D);

    // ---- the ring's loads. Wave w copies one tile per step: K (w < 2) or V, of the even
    // (w even) or odd key block. Batch u (issued in step u) fills slot (u + 2) % 3 with K of
    // stage u + 2 and V of stage u + 1. Key blocks past the last one load the last one (a
    // valid address; nobody reads them); in a ragged last block, rows past T repeat row
    // T - 1 (finite data; those keys are masked for every real query).
    const int dma_v = wave >> 1, dma_par = wave & 1;
    const int ld_slot = lane % (C::kRow / 16);
    auto ld_row = [&](int e) CGQA_INLINE { return C::kRowsPerChunk * e + lane / (C::kRow / 16); };
    auto ld_chunk_b = [&](int e) CGQA_INLINE { return (unsigned)((ld_slot ^ chunk_swizzle<D>(ld_row(e))) * 16); };
    // The swizzle of chunk e repeats every kPer chunks (rows advance by 16 between
    // repeats), so kPer lane offsets and a scalar row step cover the tile.
    constexpr int kPer = D == 64 ? 2 : 4;
    static_assert(C::kRowsPerChunk * kPer == 16 && C::kChunks % kPer == 0, "swizzle period");
    unsigned ld_off[kPer];
#pragma unroll
    for (int e = 0; e < kPer; ++e) ld_off[e] = (unsigned)ld_row(e) * kv_row_bytes + ld_chunk_b(e);
    const unsigned lds0 = __builtin_amdgcn_readfirstlane(
        (unsigned)(uintptr_t)(const __attribute__((address_space(3))) char*)smem);
    const unsigned dma_lds = lds0 + (unsigned)((2 * dma_v + dma_par) * C::kTile);
    const char* const dma_src = dma_v ? vbase : kbase;
    auto issue_batch = [&](int u) CGQA_INLINE {
        const int stage = dma_v ? u + 1 : u + 2;
        const int kb = min(max(2 * stage + dma_par, 0), nkb - 1);
        const unsigned dst = dma_lds + (unsigned)(((u + 2) % 3) * C::kSlot);
        const int row0 = 32 * kb;
        if (row0 + 32 <= T) {
            const char* base = dma_src + (size_t)row0 * kv_row_bytes;
#pragma unroll
            for (int e = 0; e < C::kChunks; ++e) {
                const unsigned o[1] = {ld_off[e % kPer]};
                load_lds16_chunks<1>(base + (size_t)(16 * (e / kPer)) * kv_row_bytes, o, dst + 1024 * e);
            }
        } else {
#pragma unroll
            for (int e = 0; e < C::kChunks; ++e) {
                const unsigned o[1] = {(unsigned)min(row0 + ld_row(e), T - 1) * kv_row_bytes + ld_chunk_b(e)};
                load_lds16_chunks<1>(dma_src, o, dst + 1024 * e);
            }
        }
    };
    // Step s: batch s - 1 (K of stage s + 1, V of stage s) complete on every wave, then
    // batch s.
    auto sync = [&](int s) CGQA_INLINE {
        wait_tiles_barrier<0>();
        issue_batch(s);
    };

    issue_batch(-2);
    issue_batch(-1);
    // Q as the B operand: lane (query n, group hl) holds dims 16*kd + 8*hl .. +7.
    bf16x8 qreg[C::kKD];
    {
        const int row = 32 * qb + n;
#pragma unroll
        for (int kd = 0; kd < C::kKD; ++kd) {
            u32x4 x = {0u, 0u, 0u, 0u};
            if (row < T) x = load16(a.q + ((size_t)b * T + row) * a.q_rs + (size_t)h * D + 16 * kd + 8 * hl);
            qreg[kd] = __builtin_bit_cast(bf16x8, x);
        }
#pragma unroll
        for (int kd = 0; kd < C::kKD; ++kd) asm volatile("" ::"v"(qreg[kd]));
    }

    // Per-lane LDS addresses of this wave's K and V tiles in slot 0: K operand row n,
    // logical chunk 2kd + hl; V operand (transposing read) rows 4*hl + j/4 (+8) of a
    // 16-row group, 8 bytes at logical column 32mb + 16*((lane>>4)&1) + 4*(j%4).
    const char* kaddr[C::kKD];
    const char* vaddr[C::kMB][2];
    {
        const int k_swz = chunk_swizzle<D>(n);
#pragma unroll
        for (int kd = 0; kd < C::kKD; ++kd) kaddr[kd] = smem + par * C::kTile + n * C::kRow + (((2 * kd + hl) ^ k_swz) << 4);
        const int v_r0 = 4 * hl + ((lane & 15) >> 2);
        const int v_swz[2] = {chunk_swizzle<D>(v_r0), chunk_swizzle<D>(v_r0 + 8)};
        const int v_chunk = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
        const int v_byte = 8 * (lane & 1);
#pragma unroll
        for (int mb = 0; mb < C::kMB; ++mb)
#pragma unroll
            for (int r = 0; r < 2; ++r)
                vaddr[mb][r] = smem + (2 + par) * C::kTile + (v_r0 + 8 * r) * C::kRow + v_byte +
                               (((4 * mb + v_chunk) ^ v_swz[r]) << 4);
    }
    // Ring offsets: K of stage t in slot t % 3, V of stage t in slot (t + 1) % 3.
    auto koff = [](int t) CGQA_INLINE { return (t % 3) * C::kSlot; };
    auto voff = [](int t) CGQA_INLINE { return ((t + 1) % 3) * C::kSlot; };

    f32x16 oacc[C::kMB];
#pragma unroll
    for (int mb = 0; mb < C::kMB; ++mb) oacc[mb] = zero16();
    float mref = 0.0f, lsum = 0.0f;

    // ---- building blocks of a step.
    auto scores = [&](int boff, f32x16& s) CGQA_INLINE {
        bf16x8 kf[C::kKD];
#pragma unroll
        for (int kd = 0; kd < C::kKD; ++kd) kf[kd] = lds_read8(kaddr[kd] + boff);
        s = mfma32x32x16(kf[0], qreg[0], zero16());
#pragma unroll
        for (int kd = 1; kd < C::kKD; ++kd) s = mfma32x32x16(kf[kd], qreg[kd], s);
    };
    // O^T += V^T P^T, 16 keys per instruction; B = P from the score registers (registers
    // 8t..8t+7 hold keys 16t + 8*(s/4) + 4*hl + s%4 for slot s), A = the same keys of V
    // read transposed.
    auto pv = [&](int boff, const bf16x8 (&pb)[2]) CGQA_INLINE {
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
            for (int mb = 0; mb < C::kMB; ++mb) oacc[mb] = mfma32x32x16(vf[t][mb], pb[t], oacc[mb]);
    };
    // Diagonal block: register i is key 8(i/4) + 4hl + i%4 against query n (same origin).
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
    auto softmax = [&](f32x16& s, bf16x8 (&pb)[2]) CGQA_INLINE {
        const float nm = -mref;
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

    f32x16 s_cur;
    bf16x8 p_prev[2];

    // One step: scores of the next block (NX), P.V of the previous one (PV), softmax of
    // the current block (masked when DG). The matrix-core work depends on neither
    // softmax, so the two interleave.
    auto step = [&](int koff_next, int voff_prev, int koff_cur, auto PVc, auto DGc, auto NXc) CGQA_INLINE {
        constexpr bool PV = decltype(PVc)::value, DG = decltype(DGc)::value, NX = decltype(NXc)::value;
        f32x16 s_nx;
        bf16x8 p_cur[2];
        if constexpr (NX) scores(koff_next, s_nx);
        if constexpr (PV) pv(voff_prev, p_prev);
        if constexpr (DG) mask_diag(s_cur);
        float t = softmax(s_cur, p_cur);
        // Code-generation workaround (as in attn_fwd.hip): keeps the compiler from merging
        // the products and the softmax with the rare-path check below.
#pragma unroll
        for (int i = 0; i < 8; ++i) {
        }
        if (wave_any(!(t <= kParRescaleLimit))) {
            // Rare: some score rose far above the reference. Recompute the block's scores,
            // move the reference to the row max and rescale what was summed so far.
            f32x16 s2;
            scores(koff_cur, s2);
            if constexpr (DG) mask_diag(s2);
            const float mnew = fmaxf(mref, row_max(s2));
            const float alpha = exp2_fast(mref - mnew);
            mref = mnew;
            lsum *= alpha;
#pragma unroll
            for (int mb = 0; mb < C::kMB; ++mb)
#pragma unroll
                for (int i = 0; i < 16; ++i) oacc[mb][i] *= alpha;
            s_cur = s2;
            t = softmax(s_cur, p_cur);
        }
        lsum += t;
        p_prev[0] = p_cur[0];
        p_prev[1] = p_cur[1];
        if constexpr (NX) s_cur = s_nx;
    };
    using F = std::false_type;
    using Tr = std::true_type;

    // ---- the wave's stages 0 .. my_len-1 (step -1 computes the first scores). Every wave
    // joins the barrier of every step -1 .. nsteps-1. Batches -2 and -1 went out before Q,
    // whose loads the compiler waited for, so step -1 only needs the barrier.
    wait_tiles_barrier<0>();
    int s_next = 0;
    if (my_len > 0) {
        scores(koff(0), s_cur);
        {
            f32x16 sm = s_cur;
            if (my_len == 1 && my_diag) mask_diag(sm);
            mref = row_max(sm);
        }
        const int s_last = my_len - 1;
        if (my_len >= 2) {
            sync(0);
            step(koff(1), 0, koff(0), F{}, F{}, Tr{});
            // Steady steps 1 .. s_last-1, unrolled by the ring period so that every LDS
            // address is a per-lane register plus an immediate.
            for (int base = 0; base < s_last; base += 3) {
                static_for<3>([&](auto Uc) CGQA_INLINE {
                    constexpr int U = decltype(Uc)::value;
                    const int s = base + U;
                    if (s < 1 || s >= s_last) return;
                    sync(s);
                    step(((U + 1) % 3) * C::kSlot, U * C::kSlot, U * C::kSlot, Tr{}, F{}, Tr{});
                });
            }
            sync(s_last);
            if (my_diag) step(0, voff(s_last - 1), koff(s_last), Tr{}, Tr{}, F{});
            else step(0, voff(s_last - 1), koff(s_last), Tr{}, F{}, F{});
        } else {
            sync(0);
            if (my_diag) step(0, 0, koff(0), F{}, Tr{}, F{});
            else step(0, 0, koff(0), F{}, F{}, F{});
        }
        pv(voff(s_last), p_prev);
        s_next = my_len;
    }
    for (; s_next < nsteps; ++s_next) sync(s_next);

    // ---- merge of the two halves of each query block: the odd-key wave writes its
    // reference max, lane sums and accumulators, the even-key wave combines them with its
    // own in that order and stores O / l and the natural-log LSE.
    wait_tiles_barrier<0>();   // every load landed, every wave done with the ring
    char* part = smem + (wave >> 1) * C::kPart;
    if (par == 1 && my_len > 0) {
#pragma unroll
        for (int mb = 0; mb < C::kMB; ++mb)
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                f32x4 x;
#pragma unroll
                for (int r = 0; r < 4; ++r) x[r] = oacc[mb][4 * u + r];
                *reinterpret_cast<f32x4*>(part + ((mb * 4 + u) * 64 + lane) * 16) = x;
            }
        reinterpret_cast<float*>(part + C::kPartO)[lane] = mref;
        reinterpret_cast<float*>(part + C::kPartO)[64 + lane] = lsum;
    }
    lds_barrier();
    if (par == 0 && my_len > 0) {
        if (qb >= 1) {   // the odd-key half has at least key block 1
            const float m1 = reinterpret_cast<const float*>(part + C::kPartO)[lane];
            const float l1 = reinterpret_cast<const float*>(part + C::kPartO)[64 + lane];
            const float mn = fmaxf(m1, mref);
            const float w1 = exp2_fast(m1 - mn), w0 = exp2_fast(mref - mn);
#pragma unroll
            for (int mb = 0; mb < C::kMB; ++mb)
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const f32x4 x = *reinterpret_cast<const f32x4*>(part + ((mb * 4 + u) * 64 + lane) * 16);
#pragma unroll
                    for (int r = 0; r < 4; ++r) oacc[mb][4 * u + r] = fmaf(x[r], w1, oacc[mb][4 * u + r] * w0);
                }
            lsum = fmaf(l1, w1, lsum * w0);
            mref = mn;
        }
        const int query = 32 * qb + n;
        if (query < T) {
            const float l = sum_halves(lsum);
            const float inv = 1.0f / l;
            uint16_t* orow = a.o + ((size_t)b * T + query) * a.o_rs + (size_t)h * D;
#pragma unroll
            for (int mb = 0; mb < C::kMB; ++mb) {
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    f32x4 x;
#pragma unroll
                    for (int r = 0; r < 4; ++r) x[r] = oacc[mb][4 * u + r] * inv;
                    const bf16x4 y = __builtin_convertvector(x, bf16x4);
                    *reinterpret_cast<u32x2*>(orow + 32 * mb + 8 * u + 4 * hl) = __builtin_bit_cast(u32x2, y);
                }
            }
            if (hl == 0) a.lse[((size_t)b * Hq + h) * T + query] = (mref + log2_fast(l)) * kLn2;
        }
    }
}

// Shapes the split kernel takes: d = 64 when the tiled kernel's grid (one workgroup per
// 128-query tile and head) would not fill one round of the chip (three workgroups on
// each of 256 CUs). There the split kernel's shorter workgroups measured faster (B8 T512
// Hq6 Hkv2: 9.4 against 10.7 us; B8 T1024: 15.7 against 17.5 us); on full grids its
// twice larger K/V traffic through LDS made it slower (B16 T1024: 27.3 against 22.2 us).
bool fwd_split_keys_chosen(const FwdArgs& a) {
    const long tiled_grid = (long)a.B * a.Hq * ((a.T + 127) / 128);
    return a.d == 64 && tiled_grid < 3 * 256;
}

hipError_t launch_fwd_split_keys(const FwdArgs& a, hipStream_t stream) {
    using C = ParCfg<64>;
    FwdArgs x = a;
    x.n_qtiles = (a.T + C::kBM - 1) / C::kBM;
    x.n_pairs = a.B * a.Hkv;
    x.xcd_group = x.n_pairs % 8 == 0 ? 1 : 0;
    const long blocks = (long)x.n_qtiles * a.B * a.Hq;
    hipLaunchKernelGGL((attn_fwd_par_kernel<64>), dim3((unsigned)blocks), dim3(C::kThreads), 0, stream, x);
    return hipGetLastError();
}

}  // namespace cgqa
