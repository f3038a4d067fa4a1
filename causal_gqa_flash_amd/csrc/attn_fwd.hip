// Forward kernel of causal grouped-query flash attention for gfx950.
//
// Method (page "A transformer in PTX", section "Flash attention"): one workgroup owns
// a block of queries of one head and walks the key blocks up to the diagonal. The
// score matrix is never written to memory: each query keeps a running max m and sum l
// (online softmax) in log2 units, the scores being multiplied once by
// scale * log2(e) and each probability being 2^(s - m). At the end O = acc / l and the
// row's log-sum-exp, converted to natural log, is saved for the backward.
//
// gfx950 design (not the page's sm_120 one):
//  * The scores are computed transposed, S^T = K Q^T, on the 32x32x16 bf16 matrix
//    core. Each lane then owns one query (a column) and 16 keys of every 32-key block,
//    so a row max or sum is an in-lane reduction plus one swap with the lane 32 away.
//  * The same accumulator registers, rounded to bf16, are the B operand of
//    O^T += V^T P^T: no trip through LDS for P (the role the pages give to their
//    C-fragment to A-fragment match). V^T comes from the row-major V tile through the
//    transposing LDS read.
//  * Q stays in registers for the whole loop. K and V tiles are staged in LDS, double
//    buffered, loaded with 16-byte global loads; rows are padded so the 16-byte row
//    reads (K) and the transposing reads (V) spread over the banks.
//  * Work order: the heaviest query blocks (the ones with the most keys) start first.
#include "cgqa_device.hpp"
#include "cgqa_launch.hpp"

namespace cgqa {

template <int D, int NQB, int BN, int NW>
struct FwdCfg {
    static constexpr int kThreads = NW * 64;
    static constexpr int kBM = NW * 32 * NQB;       // queries per workgroup
    static constexpr int kKD = D / 16;              // k-steps over the head dimension
    static constexpr int kNKB = BN / 32;            // 32-key blocks per tile
    static constexpr int kMB = D / 32;              // 32-dim blocks of the output
    static constexpr int kKPitch = D * 2 + 16;      // bytes per K row in LDS
    static constexpr int kVPitch = D * 2 + 32;      // bytes per V row in LDS
    static constexpr int kKBytes = BN * kKPitch;
    static constexpr int kVBytes = BN * kVPitch;
    static constexpr int kStage = kKBytes + kVBytes;
    static constexpr int kLds = 2 * kStage;
    static constexpr int kChunks = BN * D / 8;      // 16-byte chunks per tile and tensor
    static constexpr int kPerThread = kChunks / kThreads;
    static_assert(D == 64 || D == 128, "head dim");
    static_assert(BN % 32 == 0 && BN >= 32, "key tile");
    static_assert(kChunks % kThreads == 0, "tile load must split evenly over the threads");
    static_assert(kLds <= 160 * 1024, "LDS budget");
};

template <int D, int NQB, int BN, int NW>
__global__ __launch_bounds__(NW * 64) void attn_fwd_kernel(FwdArgs a) {
    using C = FwdCfg<D, NQB, BN, NW>;
    __shared__ __attribute__((aligned(16))) char smem[C::kLds];

    const int T = a.T, Hq = a.Hq, Hkv = a.Hkv;
    const int bh_count = a.B * Hq;
    const int bid = blockIdx.x;
    const int qt = a.n_qtiles - 1 - bid / bh_count;   // heaviest query block first
    const int bh = bid % bh_count;
    const int b = bh / Hq, h = bh % Hq;
    const int g = h / (Hq / Hkv);

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int n = lane & 31, hl = lane >> 5;
    const int q0 = qt * C::kBM;
    const int qw = q0 + wave * 32 * NQB;   // first query of this wave

    const size_t q_stride = (size_t)Hq * D;     // elements between consecutive t
    const size_t kv_stride = (size_t)Hkv * D;
    const uint16_t* qbase = a.q + ((size_t)b * T * Hq + h) * D;
    const uint16_t* kbase = a.k + ((size_t)b * T * Hkv + g) * D;
    const uint16_t* vbase = a.v + ((size_t)b * T * Hkv + g) * D;

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

    f32x16 oacc[NQB][C::kMB];
    float m_run[NQB], l_run[NQB];
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
        m_run[qb] = -INFINITY;
        l_run[qb] = 0.0f;
#pragma unroll
        for (int mb = 0; mb < C::kMB; ++mb) oacc[qb][mb] = zero16();
    }

    const int kv_end = min(T, q0 + C::kBM);            // keys 0 .. kv_end-1 are needed
    const int ntiles = (kv_end + BN - 1) / BN;

    // Cooperative tile loader: chunk c -> row c / (D/8), 16-byte column c % (D/8).
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
        char* vs = ks + C::kKBytes;
#pragma unroll
        for (int i = 0; i < C::kPerThread; ++i) {
            const int c = tid + i * C::kThreads;
            const int row = c / (D / 8), col = c % (D / 8);
            store16(ks + row * C::kKPitch + col * 16, kst[i]);
            store16(vs + row * C::kVPitch + col * 16, vst[i]);
        }
    };

    load_tile(0);
    store_tile(0);
    __syncthreads();

    // Per-lane constants of the transposing V read (see cgqa_device.hpp): lane j of its
    // 16-lane group points at row j/4 of a 4-row block and at column 4*(j%4) of the
    // group's 16 dims (groups 1 and 3 take dims 16..31 of each 32-dim block).
    const int tr_row = (lane & 15) >> 2;
    const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);

    for (int jt = 0; jt < ntiles; ++jt) {
        const int j0 = jt * BN;
        if (jt + 1 < ntiles) load_tile(j0 + BN);
        const char* ks = smem + (jt & 1) * C::kStage;
        const char* vs = ks + C::kKBytes;

        if (qw + 32 * NQB - 1 >= j0) {   // some query of this wave sees some key here
            // ---- S^T = K Q^T : rows are keys (A from LDS), columns are queries.
            f32x16 s[C::kNKB][NQB];
#pragma unroll
            for (int kb = 0; kb < C::kNKB; ++kb) {
#pragma unroll
                for (int qb = 0; qb < NQB; ++qb) s[kb][qb] = zero16();
#pragma unroll
                for (int kd = 0; kd < C::kKD; ++kd) {
                    const bf16x8 ka = lds_read8(ks + (32 * kb + n) * C::kKPitch + (16 * kd + 8 * hl) * 2);
#pragma unroll
                    for (int qb = 0; qb < NQB; ++qb) s[kb][qb] = mfma32x32x16(ka, qreg[qb][kd], s[kb][qb]);
                }
            }
            // ---- online softmax in log2 units, one query per lane.
            const bool need_mask = (j0 + BN - 1 > qw);
#pragma unroll
            for (int qb = 0; qb < NQB; ++qb) {
                const int query = qw + 32 * qb + n;
                float mx = -INFINITY;
#pragma unroll
                for (int kb = 0; kb < C::kNKB; ++kb) {
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        float x = s[kb][qb][i] * a.scale_log2;
                        if (need_mask) {
                            const int key = j0 + 32 * kb + 8 * (i >> 2) + 4 * hl + (i & 3);
                            if (key > query) x = -INFINITY;
                        }
                        s[kb][qb][i] = x;
                        mx = fmaxf(mx, x);
                    }
                }
                mx = fmaxf(mx, swap_halves(mx));
                const float m_new = fmaxf(m_run[qb], mx);   // finite: key 0 came first
                const float alpha = exp2_fast(m_run[qb] - m_new);
                float sum = 0.0f;
#pragma unroll
                for (int kb = 0; kb < C::kNKB; ++kb) {
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        const float p = exp2_fast(s[kb][qb][i] - m_new);
                        s[kb][qb][i] = p;
                        sum += p;
                    }
                }
                sum += swap_halves(sum);
                l_run[qb] = l_run[qb] * alpha + sum;
                m_run[qb] = m_new;
#pragma unroll
                for (int mb = 0; mb < C::kMB; ++mb)
#pragma unroll
                    for (int i = 0; i < 16; ++i) oacc[qb][mb][i] *= alpha;
            }
            // ---- O^T += V^T P^T, 16 keys per instruction. B = P straight from the score
            // registers: registers 8t..8t+7 of a 32-key block hold keys
            // 16t + 8*(s/4) + 4*hl + s%4 for slot s. A = the same keys of V, read
            // transposed: slots 0..3 from rows 16t + 4*hl + r, slots 4..7 from rows
            // 16t + 8 + 4*hl + r.
#pragma unroll
            for (int kb = 0; kb < C::kNKB; ++kb) {
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    bf16x8 pb[NQB];
#pragma unroll
                    for (int qb = 0; qb < NQB; ++qb) pb[qb] = t == 0 ? pack_lo(s[kb][qb]) : pack_hi(s[kb][qb]);
                    const int r0 = 32 * kb + 16 * t + 4 * hl + tr_row;
#pragma unroll
                    for (int mb = 0; mb < C::kMB; ++mb) {
                        const char* p0 = vs + r0 * C::kVPitch + (32 * mb + tr_col) * 2;
                        const bf16x8 va = concat(lds_read_tr4(p0), lds_read_tr4(p0 + 8 * C::kVPitch));
#pragma unroll
                        for (int qb = 0; qb < NQB; ++qb) oacc[qb][mb] = mfma32x32x16(va, pb[qb], oacc[qb][mb]);
                    }
                }
            }
        }
        if (jt + 1 < ntiles) store_tile((jt + 1) & 1);
        __syncthreads();
    }

    // ---- epilogue: O = acc / l in bf16, LSE = ln2 * (m + log2 l).
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
        const int query = qw + 32 * qb + n;
        if (query >= T) continue;
        const float inv = 1.0f / l_run[qb];
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
        if (hl == 0) a.lse[((size_t)b * Hq + h) * T + query] = (m_run[qb] + log2_fast(l_run[qb])) * kLn2;
    }
}

template <int D, int NQB, int BN, int NW>
static hipError_t launch_fwd_t(const FwdArgs& a, hipStream_t stream) {
    using C = FwdCfg<D, NQB, BN, NW>;
    FwdArgs x = a;
    x.n_qtiles = (a.T + C::kBM - 1) / C::kBM;
    const long blocks = (long)x.n_qtiles * a.B * a.Hq;
    hipLaunchKernelGGL((attn_fwd_kernel<D, NQB, BN, NW>), dim3((unsigned)blocks), dim3(C::kThreads), 0,
                       stream, x);
    return hipGetLastError();
}

hipError_t launch_fwd(const FwdArgs& a, hipStream_t stream) {
    if (a.d == 64) return launch_fwd_t<64, 1, 64, 4>(a, stream);
    return launch_fwd_t<128, 1, 64, 4>(a, stream);
}

}  // namespace cgqa
