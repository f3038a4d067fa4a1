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
//  * The reference max is not updated tile by tile. Softmax is invariant to the
//    reference (O = sum p v / sum p and LSE = m + log2 l hold for any m), so m is taken
//    from the first key block (which holds key 0 for every query) and kept while every
//    probability stays below 2^40. Only when a block's sum shows a larger value (a
//    score 40 log2 units above m) does the wave recompute that block's scores, move m
//    to the new row max and rescale l and the accumulators. This keeps the per-score
//    max and the per-block rescale off the vector ALU, which limits this kernel at
//    d = 64: one exp2, one fma, one add and half a convert per score remain.
//  * K and V tiles go straight from global memory to LDS (global_load_lds_dwordx4, no
//    staging registers) into a ring of three stages, two tiles ahead of the compute.
//    A direct load writes 1 KB of consecutive LDS per instruction, so rows cannot be
//    padded; instead the 16-byte chunks of each row are XOR-swizzled (see
//    chunk_swizzle) so that both the 16-byte row reads of K and the transposing reads
//    of V spread over the 64 banks.
//  * Work order: the heaviest query blocks (the ones with the most keys) start first.
#include "cgqa_device.hpp"
#include "cgqa_launch.hpp"

#include <string.h>

#include <type_traits>
#include <vector>

namespace cgqa {

template <int D, int NQB, int BN, int NW>
struct FwdCfg {
    static constexpr int kThreads = NW * 64;
    static constexpr int kBN = BN;                  // keys per tile
    static constexpr int kBM = NW * 32 * NQB;       // queries per workgroup
    static constexpr int kKD = D / 16;              // k-steps over the head dimension
    static constexpr int kNKB = kBN / 32;           // 32-key blocks per tile
    static constexpr int kMB = D / 32;              // 32-dim blocks of the output
    static constexpr int kRow = D * 2;              // bytes per K or V row in LDS
    static constexpr int kTile = kBN * kRow;        // bytes per K (or V) tile
    static constexpr int kStages = 3;
    static constexpr int kStage = 2 * kTile;        // K then V
    static constexpr int kLds = kStages * kStage;
    static constexpr int kLoadsPerTensor = kTile / 1024 / NW;   // 1 KB per wave instruction
    static constexpr int kLoadsPerTile = 2 * kLoadsPerTensor;    // per wave
    static constexpr int kRowsPerLoad = 1024 / kRow;
    static_assert(D == 64 || D == 128, "head dim");
    static_assert(kTile % (1024 * NW) == 0, "tile load must split evenly over the waves");
    static_assert(kLds <= 160 * 1024, "LDS budget");
};

// Probabilities above this trigger a move of the reference max.
constexpr float kRescaleLimit = 1099511627776.0f;   // 2^40

template <int D, int NQB, int BN, int NW>
__global__ __launch_bounds__(NW * 64) void attn_fwd_kernel(FwdArgs a) {
    using C = FwdCfg<D, NQB, BN, NW>;
    __shared__ __attribute__((aligned(1024))) char smem[C::kLds];

    const int T = a.T, Hq = a.Hq, Hkv = a.Hkv;
    const int bh_count = a.B * Hq;
    // Task t: query tile n_qtiles-1 - t / bh_count of (batch, head) t % bh_count, so the
    // default order starts the heaviest tiles first; small grids use the host's map.
    const int task = a.use_map ? (int)a.task_map[blockIdx.x] : (int)blockIdx.x;
    const int qt = a.n_qtiles - 1 - task / bh_count;
    const int bh = task % bh_count;
    const int b = bh / Hq, h = bh % Hq;
    const int g = h / (Hq / Hkv);

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int n = lane & 31, hl = lane >> 5;
    const int q0 = qt * C::kBM;
    const int qw = q0 + wave * 32 * NQB;   // first query of this wave
    const float c = a.scale_log2;

    const size_t q_stride = (size_t)Hq * D;     // elements between consecutive t
    const size_t kv_stride = (size_t)Hkv * D;
    const uint16_t* qbase = a.q + ((size_t)b * T * Hq + h) * D;
    const uint16_t* kbase = a.k + ((size_t)b * T * Hkv + g) * D;
    const uint16_t* vbase = a.v + ((size_t)b * T * Hkv + g) * D;

    const int kv_end = min(T, q0 + C::kBM);            // keys 0 .. kv_end-1 are needed
    const int ntiles = (kv_end + C::kBN - 1) / C::kBN;

    // Tile loader: wave instruction i of this wave fills rows
    // kRowsPerLoad * (wave * kLoadsPerTensor + i) + lane / (kRow/16) of the tile, slot
    // lane % (kRow/16), with the logical chunk that the swizzle puts there. Rows past
    // T read row T-1 (finite data; those keys are masked for every real query).
    const int ld_slot = lane % (C::kRow / 16);
    int ld_row[C::kLoadsPerTensor], ld_chunk[C::kLoadsPerTensor];
#pragma unroll
    for (int i = 0; i < C::kLoadsPerTensor; ++i) {
        ld_row[i] = C::kRowsPerLoad * (wave * C::kLoadsPerTensor + i) + lane / (C::kRow / 16);
        ld_chunk[i] = ld_slot ^ chunk_swizzle<D>(ld_row[i]);
    }
    auto issue_tile = [&](int stage, int jt) {
        char* ks = smem + stage * C::kStage;
        char* vs = ks + C::kTile;
#pragma unroll
        for (int i = 0; i < C::kLoadsPerTensor; ++i) {
            const int key = min(jt * C::kBN + ld_row[i], T - 1);
            const size_t off = (size_t)key * kv_stride + ld_chunk[i] * 8;
            const int dst = (wave * C::kLoadsPerTensor + i) * 1024;
            load_lds16(kbase + off, ks + dst);
            load_lds16(vbase + off, vs + dst);
        }
    };

    issue_tile(0, 0);
    if (ntiles > 1) issue_tile(1, 1);

    // Q as the B operand: lane (query n, group hl) holds dims 16*kd + 8*hl .. +7.
    bf16x8 qreg[NQB][C::kKD];
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
        const int row = qw + 32 * qb + n;
#pragma unroll
        for (int kd = 0; kd < C::kKD; ++kd) {
            u32x4 x = {0u, 0u, 0u, 0u};
            if (row < T) x = load16(qbase + (size_t)row * q_stride + 16 * kd + 8 * hl);
            qreg[qb][kd] = __builtin_bit_cast(bf16x8, x);
        }
    }

    // Q in registers before the loop on every path, so the compiler's waits for it do
    // not land inside the loop (where they would also wait for the tile prefetch).
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
        for (int kd = 0; kd < C::kKD; ++kd) asm volatile("" ::"v"(qreg[qb][kd]));

    f32x16 oacc[NQB][C::kMB];
    float mref[NQB], lsum[NQB];
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
        mref[qb] = 0.0f;
        lsum[qb] = 0.0f;
#pragma unroll
        for (int mb = 0; mb < C::kMB; ++mb) oacc[qb][mb] = zero16();
    }

    // Per-lane LDS offsets. K operand: row 32kb + n, logical chunk 2kd + hl. V operand
    // (transposing read): lane j of its 16-lane group reads row 4*hl + j/4 (+8 for the
    // second half) of a 16-row group, 8 bytes at logical column
    // 32mb + 16*((lane>>4)&1) + 4*(j%4). Rows only enter the swizzle through r % 16,
    // which does not depend on the block, so these are per-lane constants.
    // With the tile loop unrolled by the stage count below, every read is one of these
    // per-lane addresses plus an immediate offset.
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

    for (int jt0 = 0; jt0 < ntiles; jt0 += C::kStages) {
      static_for<C::kStages>([&](auto Uc) {
        constexpr int U = decltype(Uc)::value;
        constexpr int soff = U * C::kStage;
        const int jt = jt0 + U;
        if (jt >= ntiles) return;
        // Tile jt is complete once at most the next tile's loads are outstanding; the
        // barrier also tells every wave that all waves are done with tile jt - 1,
        // whose stage the loads of tile jt + 2 reuse.
        if (jt + 1 < ntiles) wait_tiles_barrier<C::kLoadsPerTile>();
        else wait_tiles_barrier<0>();
        if (jt + 2 < ntiles) issue_tile((U + 2) % C::kStages, jt + 2);

        const int j0 = jt * C::kBN;

        if (qw + 32 * NQB - 1 < j0) return;   // every query of this wave is before the tile
#pragma unroll
        for (int kb = 0; kb < C::kNKB; ++kb) {
            const int jb = j0 + 32 * kb;
            if (qw + 32 * NQB - 1 < jb) break;      // the rest of the tile is masked
            // S^T = K Q^T (rows: keys, A from LDS; columns: queries), masked above the
            // diagonal. Register i of block qb is key jb + 8(i/4) + 4hl + i%4.
            f32x16 s[NQB];
            const bool need_mask = (jb + 31 > qw);
            const int koff = soff + 32 * kb * C::kRow;
            auto scores = [&]() {
#pragma unroll
                for (int qb = 0; qb < NQB; ++qb) s[qb] = zero16();
#pragma unroll
                for (int kd = 0; kd < C::kKD; ++kd) {
                    const bf16x8 ka = lds_read8(kaddr[kd] + koff);
#pragma unroll
                    for (int qb = 0; qb < NQB; ++qb) s[qb] = mfma32x32x16(ka, qreg[qb][kd], s[qb]);
                }
                if (need_mask) {
#pragma unroll
                    for (int qb = 0; qb < NQB; ++qb) {
                        const int rel = jb + 4 * hl - (qw + 32 * qb + n);   // key - query at i = 0
#pragma unroll
                        for (int i = 0; i < 16; ++i)
                            if (rel + 8 * (i >> 2) + (i & 3) > 0) s[qb][i] = -INFINITY;
                    }
                }
            };
            auto row_max = [&](int qb) {
                float mx = -INFINITY;
#pragma unroll
                for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[qb][i]);
                mx = fmaxf(mx, swap_halves(mx));
                return mx * c;
            };
            float tsum[NQB];
            auto exponentials = [&]() {
#pragma unroll
                for (int qb = 0; qb < NQB; ++qb) {
                    tsum[qb] = 0.0f;
                    const float nm = -mref[qb];
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        const float p = exp2_fast(fmaf(s[qb][i], c, nm));
                        s[qb][i] = p;
                        tsum[qb] += p;
                    }
                }
            };

            scores();
            if (jb == 0) {
                // Key 0 is in this block for every query: a finite reference max.
#pragma unroll
                for (int qb = 0; qb < NQB; ++qb) mref[qb] = row_max(qb);
            }
            exponentials();
            bool big = false;
#pragma unroll
            for (int qb = 0; qb < NQB; ++qb) big |= !(tsum[qb] <= kRescaleLimit);
            if (wave_any(big)) {
                // Rare: some score rose far above the reference. Recompute the block's
                // scores, move the reference to the row max and rescale what was
                // summed so far.
                scores();
#pragma unroll
                for (int qb = 0; qb < NQB; ++qb) {
                    const float mnew = fmaxf(mref[qb], row_max(qb));
                    const float alpha = exp2_fast(mref[qb] - mnew);
                    mref[qb] = mnew;
                    lsum[qb] *= alpha;
#pragma unroll
                    for (int mb = 0; mb < C::kMB; ++mb)
#pragma unroll
                        for (int i = 0; i < 16; ++i) oacc[qb][mb][i] *= alpha;
                }
                exponentials();
            }
#pragma unroll
            for (int qb = 0; qb < NQB; ++qb) lsum[qb] += tsum[qb];

            // O^T += V^T P^T, 16 keys per instruction. B = P straight from the score
            // registers: registers 8t..8t+7 hold keys 16t + 8*(s/4) + 4*hl + s%4 for
            // slot s. A = the same keys of V, read transposed: slots 0..3 from rows
            // 16t + 4*hl + r, slots 4..7 from rows 16t + 8 + 4*hl + r.
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                bf16x8 pb[NQB];
#pragma unroll
                for (int qb = 0; qb < NQB; ++qb) pb[qb] = t == 0 ? pack_lo(s[qb]) : pack_hi(s[qb]);
                const int voff = soff + (32 * kb + 16 * t) * C::kRow;
#pragma unroll
                for (int mb = 0; mb < C::kMB; ++mb) {
                    const bf16x8 va = concat(lds_read_tr4(vaddr[mb][0] + voff), lds_read_tr4(vaddr[mb][1] + voff));
#pragma unroll
                    for (int qb = 0; qb < NQB; ++qb) oacc[qb][mb] = mfma32x32x16(va, pb[qb], oacc[qb][mb]);
                }
            }
        }
      });
    }

    // ---- epilogue: O = acc / l in bf16, LSE = ln2 * (m + log2 l).
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
        const int query = qw + 32 * qb + n;
        const float l = lsum[qb] + swap_halves(lsum[qb]);
        if (query >= T) continue;
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
}

// Balanced placement for grids of at most three workgroups per CU. All of them are
// resident at once, and the dispatcher places workgroup x on CU x mod n_cu (measured on
// MI355X: x, x + 256 and x + 512 share a CU). A task's load is proportional to its
// number of key tiles, n_qtiles - t / bh_count; the longest tasks are dealt first,
// each to the least loaded CU with a free slot. A different placement only costs
// balance, never correctness.
static bool build_task_map(int blocks, int bh_count, int n_qtiles, int n_cu, uint16_t* map) {
    if (n_cu <= 0 || blocks > kFwdMaxMapped || blocks > 3 * n_cu || blocks <= n_cu) return false;
    struct Cache { int blocks = -1, bh = -1, nq = -1, ncu = -1; uint16_t map[kFwdMaxMapped]; };
    thread_local Cache cache;
    if (cache.blocks == blocks && cache.bh == bh_count && cache.nq == n_qtiles && cache.ncu == n_cu) {
        memcpy(map, cache.map, sizeof(uint16_t) * blocks);
        return true;
    }
    std::vector<int> load(n_cu, 0), used(n_cu, 0);
    // Tasks are already in decreasing load order (t increases as the tile gets lighter).
    for (int t = 0; t < blocks; ++t) {
        const int w = n_qtiles - t / bh_count;
        int best = -1;
        for (int c = 0; c < n_cu; ++c) {
            if (c + used[c] * n_cu >= blocks) continue;   // no free slot on this CU
            if (best < 0 || load[c] < load[best]) best = c;
        }
        map[best + used[best] * n_cu] = (uint16_t)t;
        ++used[best];
        load[best] += w;
    }
    cache.blocks = blocks;
    cache.bh = bh_count;
    cache.nq = n_qtiles;
    cache.ncu = n_cu;
    memcpy(cache.map, map, sizeof(uint16_t) * blocks);
    return true;
}

static int device_cu_count() {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    return n;
}

template <int D, int NQB, int BN, int NW>
static hipError_t launch_fwd_t(const FwdArgs& a, hipStream_t stream) {
    using C = FwdCfg<D, NQB, BN, NW>;
    FwdArgs x = a;
    x.n_qtiles = (a.T + C::kBM - 1) / C::kBM;
    const long blocks = (long)x.n_qtiles * a.B * a.Hq;
    x.use_map = blocks <= kFwdMaxMapped &&
                build_task_map((int)blocks, a.B * a.Hq, x.n_qtiles, device_cu_count(), x.task_map);
    hipLaunchKernelGGL((attn_fwd_kernel<D, NQB, BN, NW>), dim3((unsigned)blocks), dim3(C::kThreads), 0, stream, x);
    return hipGetLastError();
}

hipError_t launch_fwd(const FwdArgs& a, hipStream_t stream) {
    if (a.d == 64) return launch_fwd_t<64, 1, 64, 4>(a, stream);
    return launch_fwd_t<128, 1, 32, 4>(a, stream);
}

}  // namespace cgqa
