// bf16 matrix product with layout flags (page "A transformer in PTX", section "Three ways
// to run it": the projections are one matmul kernel that takes flags for operands stored
// the other way round, reads those tiles with a transposing load instead of transposing
// memory, gives the same bits as pre-transposed data, and can start its accumulators
// from an existing result to add into it; page "Talking to the GPU", the tensor-core
// matmul: block tiles staged through shared memory in stages).
//
//   C[m][n] = sum_k A[m][k] B[n][k]  (+ R[m][n])
//
// A is stored [M][K] or, with the A_KM flag, [K][M]; B is stored [N][K] (a weight matrix
// as a projection x W^T uses it) or, with B_KN, [K][N]. Products accumulate in fp32 on
// the 32x32x16 bf16 matrix core, k ascending in steps of 16, starting from R (fp32, may
// be C itself) or zero; C is fp32 or bf16 (round to nearest even).
//
// gfx950 design: a workgroup of four waves owns a 128 x 128 tile of C, each wave a
// 64 x 64 quarter (2 x 2 blocks of 32 x 32). K advances 32 at a time through a 3-stage
// LDS ring filled by direct-to-LDS loads two tiles ahead; the loop is matrix-core and
// LDS work only. Tiles of an operand stored [rows][K] are 128 rows of 64 bytes; tiles of
// one stored [K][rows] are 32 rows of 256 bytes, read into the same register fragment by
// the transposing LDS read (ds_read_b64_tr_b16), so both layouts feed the matrix core
// identical values in identical order. Workgroups that share a row block of A run on
// one XCD, whose L2 then serves that block to all of them.
//
// Shapes with few output tiles and a long K (dW = dy^T x: 15 tiles, K = 16384) leave
// most of the chip idle; given a workspace, the K range is split over S workgroups per
// tile, each writing its fp32 partial product, and a second kernel adds the S partials
// in split order (and R) into C. The split count is a function of M, N, K and the
// workspace size only, so results are repeatable.
#include <mutex>

#include "cgqa_device.hpp"
#include "cgqa_launch.hpp"

namespace cgqa {
namespace {

constexpr int kBM = 128, kBN = 128, kBK = 32;
constexpr int kThreads = 256;
constexpr int kStages = 3;
constexpr int kTileBytes = 128 * kBK * 2;          // 8 KB per operand and stage
constexpr int kStageBytes = 2 * kTileBytes;        // A then B
constexpr int kLds = kStages * kStageBytes;        // 48 KB: three workgroups per CU

// Physical 16-byte slot of logical chunk c (8 k values) in row r of a [rows][32 k] tile:
// 16 lanes reading one chunk of 16 consecutive rows hit 16 distinct slots of a 256-byte
// bank window.
__device__ __forceinline__ int rk_swizzle(int r) { return (r >> 2) & 3; }

// Per-lane DMA offsets of one operand: wave w fills 1 KB pieces 2w and 2w+1 of each tile.
// Rows past the matrix read its last row (or chunk): finite data whose products land in
// rows or columns of C that are not stored.
template <bool KMAJOR>
struct Loader {
    unsigned off[2];      // bytes from the operand's base at k0 = 0
    unsigned kstep;       // bytes the base moves per 32-k tile
    __device__ void init(int wave, int lane, int rows, int K, int r0) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int e = 2 * wave + i;
            if constexpr (!KMAJOR) {
                const int row = 16 * e + (lane >> 2);
                const int c = (lane & 3) ^ rk_swizzle(row);
                const int gr = min(r0 + row, rows - 1);
                off[i] = (unsigned)gr * (unsigned)K * 2u + (unsigned)c * 16u;
            } else {
                const int row = 4 * e + (lane >> 4);
                const int c = (lane & 15) ^ chunk_swizzle<128>(row);
                const int col = min(r0 + 8 * c, rows - 8);
                off[i] = (unsigned)row * (unsigned)rows * 2u + (unsigned)col * 2u;
            }
        }
        kstep = KMAJOR ? (unsigned)kBK * (unsigned)rows * 2u : (unsigned)kBK * 2u;
    }
    // Tile kt of the operand into LDS byte address `lds` (wave-uniform). One load per
    // 1 KB piece, each with its own full offset (no instruction offset, so the unsigned
    // lane offset is never reduced below zero).
    __device__ void issue(const uint16_t* base, int kt, int wave, unsigned lds) const {
        const char* b = reinterpret_cast<const char*>(base) + (size_t)kt * kstep;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const unsigned o[1] = {off[i]};
            load_lds16_chunks<1>(b, o, lds + 2048u * (unsigned)wave + 1024u * (unsigned)i);
        }
    }
};

// Register fragment of block `blk` (32 rows) and k-step t (16 k) from a tile in LDS:
// lane l holds row l % 32, k = 16t + 8*(l/32) + s in slot s, for either layout (the
// matrix core pairs slot s of A with slot s of B, so both operands must use one order).
template <bool KMAJOR>
struct Frag {
    const char* addr[2][2];   // [block of the wave][t (row-major) or r (k-major)]
    __device__ void init(const char* tile, int lane, int first_row) {
        const int n = lane & 31, hl = lane >> 5;
        if constexpr (!KMAJOR) {
#pragma unroll
            for (int bi = 0; bi < 2; ++bi) {
                const int row = first_row + 32 * bi + n;
#pragma unroll
                for (int t = 0; t < 2; ++t)
                    addr[bi][t] = tile + row * 64 + (((2 * t + hl) ^ rk_swizzle(row)) << 4);
            }
        } else {
            // Transposing read: lane j of a 16-lane group points at row 8*hl + j/4 (then
            // +4) of a 16-row group, 8 bytes at column 32*blk + 16*((lane>>4)&1) + 4*(j%4);
            // the read hands lane j that column for the 4 rows, so slots 0-3 hold k =
            // 8*hl + 0..3 and slots 4-7 k = 8*hl + 4..7.
            const int v_r0 = 8 * hl + ((lane & 15) >> 2);
            const int v_swz[2] = {chunk_swizzle<128>(v_r0), chunk_swizzle<128>(v_r0 + 4)};
            const int v_chunk = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
            const int v_byte = 8 * (lane & 1);
#pragma unroll
            for (int bi = 0; bi < 2; ++bi) {
                const int mb = first_row / 32 + bi;
#pragma unroll
                for (int r = 0; r < 2; ++r)
                    addr[bi][r] = tile + (v_r0 + 4 * r) * 256 + v_byte + (((4 * mb + v_chunk) ^ v_swz[r]) << 4);
            }
        }
    }
    template <int BI, int T>
    __device__ bf16x8 read(int stage_off) const {
        if constexpr (!KMAJOR) return lds_read8(addr[BI][T] + stage_off);
        else
            return concat(lds_read_tr4(addr[BI][0] + stage_off + 16 * T * 256),
                          lds_read_tr4(addr[BI][1] + stage_off + 16 * T * 256));
    }
};

template <bool AKM, bool BKN>
__global__ __launch_bounds__(kThreads, 3) void gemm_bf16_kernel(GemmArgs a) {
    __shared__ __attribute__((aligned(1024))) char smem[kLds];
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    // Tile and K split of this workgroup: row blocks tm with tm % 8 == xcd run on XCD
    // xcd; splits are the slowest index.
    const int xcd = (int)blockIdx.x & 7, local = (int)blockIdx.x >> 3;
    const int per = (a.tiles_m + 7) / 8 * a.tiles_n;
    const int split = local / per, l2 = local % per;
    const int tm = xcd + 8 * (l2 / a.tiles_n), tn = l2 % a.tiles_n;
    if (tm >= a.tiles_m) return;
    const int m0 = tm * kBM, n0 = tn * kBN;
    const int wm = wave >> 1, wn = wave & 1;           // 64 x 64 quarter of the tile
    const int kt0 = split * a.kps;                     // this split's 32-k tiles
    const int nk = min(a.K / kBK - kt0, a.kps);

    Loader<AKM> la;
    Loader<BKN> lb;
    la.init(wave, lane, a.M, a.K, m0);
    lb.init(wave, lane, a.N, a.K, n0);
    const unsigned lds0 = __builtin_amdgcn_readfirstlane(
        (unsigned)(uintptr_t)(const __attribute__((address_space(3))) char*)smem);
    // Tile kt (counted from this split's first) into stage kt % 3.
    auto issue = [&](int kt) CGQA_INLINE {
        const unsigned st = lds0 + (unsigned)(kt % kStages) * kStageBytes;
        la.issue(a.a, kt0 + kt, wave, st);
        lb.issue(a.b, kt0 + kt, wave, st + kTileBytes);
    };
    Frag<AKM> fa;
    Frag<BKN> fb;
    fa.init(smem, lane, 64 * wm);
    fb.init(smem + kTileBytes, lane, 64 * wn);

    // Element (bi, bj, i) of this lane: row 8(i/4) + 4*half + i%4 of block bi, column
    // l % 32 of block bj.
    const int n_l = lane & 31, hl = lane >> 5;
    auto row_of = [&](int bi, int i) CGQA_INLINE { return m0 + 64 * wm + 32 * bi + 8 * (i >> 2) + 4 * hl + (i & 3); };
    auto col_of = [&](int bj) CGQA_INLINE { return n0 + 64 * wn + 32 * bj + n_l; };

    // The accumulators start from R (without a K split; with one, the sum adds R): the
    // loads go out before the first tiles, and elements outside C read a clamped one.
    f32x16 acc[2][2];
#pragma unroll
    for (int bi = 0; bi < 2; ++bi)
#pragma unroll
        for (int bj = 0; bj < 2; ++bj) {
            if (a.r && a.ksplit == 1) {
                const int n = min(col_of(bj), a.N - 1);
#pragma unroll
                for (int i = 0; i < 16; ++i) acc[bi][bj][i] = a.r[(size_t)min(row_of(bi, i), a.M - 1) * a.N + n];
            } else {
                acc[bi][bj] = zero16();
            }
        }

    if (nk > 0) issue(0);
    if (nk > 1) issue(1);
    // Stages cycle with period 3: unrolled so every LDS offset is an immediate.
    for (int k0 = 0; k0 < nk; k0 += kStages) {
        static_for<kStages>([&](auto Sc) CGQA_INLINE {
            constexpr int S = decltype(Sc)::value;
            const int kt = k0 + S;
            if (kt >= nk) return;
            // Tile kt complete for every wave (tile kt+1 may stay in flight: four loads
            // per wave and tile); the stage of tile kt-1 is free after this barrier.
            if (kt + 1 < nk) wait_tiles_barrier<4>();
            else wait_tiles_barrier<0>();
            if (kt + 2 < nk) issue(kt + 2);
            constexpr int so = S * kStageBytes;
            static_for<2>([&](auto Tc) CGQA_INLINE {
                constexpr int T = decltype(Tc)::value;
                const bf16x8 a0 = fa.template read<0, T>(so), a1 = fa.template read<1, T>(so);
                const bf16x8 b0 = fb.template read<0, T>(so), b1 = fb.template read<1, T>(so);
                acc[0][0] = mfma32x32x16(a0, b0, acc[0][0]);
                acc[0][1] = mfma32x32x16(a0, b1, acc[0][1]);
                acc[1][0] = mfma32x32x16(a1, b0, acc[1][0]);
                acc[1][1] = mfma32x32x16(a1, b1, acc[1][1]);
            });
        });
    }

    // Epilogue: with a K split the fp32 partial goes to the workspace slice of this split.
    float* const part = a.ksplit > 1 ? a.ws + (size_t)split * gemm_slice_floats(a.M, a.N) : nullptr;
    const bool full = m0 + kBM <= a.M && n0 + kBN <= a.N;   // no bounds checks needed
#pragma unroll
    for (int bi = 0; bi < 2; ++bi)
#pragma unroll
        for (int bj = 0; bj < 2; ++bj) {
            const int n = col_of(bj);
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int m = row_of(bi, i);
                if (!full && (m >= a.M || n >= a.N)) continue;
                const size_t idx = (size_t)m * a.N + n;
                const float x = acc[bi][bj][i];
                if (part) {
                    part[idx] = x;
                } else if (a.c_bf16) {
                    const uint32_t u = __float_as_uint(x);
                    static_cast<uint16_t*>(a.c)[idx] = (uint16_t)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
                } else {
                    static_cast<float*>(a.c)[idx] = x;
                }
            }
        }
}

// C = sum over splits s = 0 .. S-1 (in order) of the partials, + R. Four consecutive
// elements per thread (slices are padded to a multiple of four floats), eight partials in
// flight; the tail of M*N that is not a whole group of four goes one element at a time.
__global__ __launch_bounds__(kThreads) void gemm_splitk_sum_kernel(GemmArgs a) {
    const size_t mn = (size_t)a.M * a.N, slice = gemm_slice_floats(a.M, a.N), n4 = mn / 4;
    const size_t stride = (size_t)gridDim.x * kThreads;
    auto finish_store = [&](float x, size_t idx) CGQA_INLINE {
        if (a.r) x += a.r[idx];
        if (a.c_bf16) {
            const uint32_t u = __float_as_uint(x);
            static_cast<uint16_t*>(a.c)[idx] = (uint16_t)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
        } else {
            static_cast<float*>(a.c)[idx] = x;
        }
    };
    for (size_t q = (size_t)blockIdx.x * kThreads + threadIdx.x; q < n4; q += stride) {
        f32x4 x = *reinterpret_cast<const f32x4*>(a.ws + 4 * q);
        int s = 1;
        for (; s + 8 <= a.ksplit; s += 8) {
            f32x4 y[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) y[u] = *reinterpret_cast<const f32x4*>(a.ws + (size_t)(s + u) * slice + 4 * q);
#pragma unroll
            for (int u = 0; u < 8; ++u) x += y[u];
        }
        for (; s < a.ksplit; ++s) x += *reinterpret_cast<const f32x4*>(a.ws + (size_t)s * slice + 4 * q);
#pragma unroll
        for (int e = 0; e < 4; ++e) finish_store(x[e], 4 * q + e);
    }
    for (size_t idx = 4 * n4 + (size_t)blockIdx.x * kThreads + threadIdx.x; idx < mn; idx += stride) {
        float x = a.ws[idx];
        for (int s = 1; s < a.ksplit; ++s) x += a.ws[(size_t)s * slice + idx];
        finish_store(x, idx);
    }
}

}  // namespace

// Splits of K: only for shapes with fewer than 256 output tiles and at least 16 tiles of
// 32 k, aiming at ~512 workgroups with at least 8 k-tiles each, at most 32 splits, and
// no more than the workspace holds. Returns 1 for no split.
int gemm_splits(int M, int N, int K, size_t ws_bytes) {
    const long tiles = (long)((M + kBM - 1) / kBM) * ((N + kBN - 1) / kBN);
    const int nk = K / kBK;
    if (tiles == 0 || tiles >= 256 || nk < 16) return 1;
    long s = (512 + tiles - 1) / tiles;
    s = s < nk / 8 ? s : nk / 8;
    s = s < 32 ? s : 32;
    const size_t per = gemm_slice_floats(M, N) * 4;
    if ((size_t)s * per > ws_bytes) s = (long)(ws_bytes / per);
    if (s < 2) return 1;
    const int kps = (nk + (int)s - 1) / (int)s;
    return (nk + kps - 1) / kps;   // no empty split
}

// Scratch of the allocation-free entry point: the split-K partials of cgqa_gemm_static
// live in this file-scope array, one copy per GPU, which the library holds until the
// process ends and which every such call on that GPU shares. In host code its name
// stands for a host-side shadow, not a device address: kernels get the address that
// hipGetSymbolAddress returns, looked up once per device (with that device current)
// and kept per device.
static __device__ __align__(256) float scratch[kGemmScratchBytes / sizeof(float)];

namespace {
constexpr int kMaxDevices = 64;
std::once_flag g_scratch_once[kMaxDevices];
float* g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];
}  // namespace

hipError_t gemm_scratch(float** ptr) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::call_once(g_scratch_once[dev], [dev] {
        void* p = nullptr;
        g_scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        g_scratch_ptr[dev] = g_scratch_err[dev] == hipSuccess ? static_cast<float*>(p) : nullptr;
    });
    if (g_scratch_err[dev] != hipSuccess) return g_scratch_err[dev];
    *ptr = g_scratch_ptr[dev];
    return hipSuccess;
}

hipError_t launch_gemm(const GemmArgs& a0, hipStream_t stream) {
    GemmArgs a = a0;
    a.tiles_m = (a.M + kBM - 1) / kBM;
    a.tiles_n = (a.N + kBN - 1) / kBN;
    const int nk = a.K / kBK;
    a.ksplit = gemm_splits(a.M, a.N, a.K, a.ws ? a.ws_bytes : 0);
    a.kps = a.ksplit > 1 ? (nk + a.ksplit - 1) / a.ksplit : nk;
    if (a.ksplit > 1) a.ksplit = (nk + a.kps - 1) / a.kps;   // every split non-empty
    // XCD x takes row blocks x, x+8, ...: 8 * ceil(tiles_m / 8) * tiles_n workgroups per
    // split, the ones past the last row block return at once.
    const long blocks = 8L * ((a.tiles_m + 7) / 8) * a.tiles_n * a.ksplit;
    const dim3 grid((unsigned)blocks), block(kThreads);
    if (!a.a_km && !a.b_kn) hipLaunchKernelGGL((gemm_bf16_kernel<false, false>), grid, block, 0, stream, a);
    else if (!a.a_km) hipLaunchKernelGGL((gemm_bf16_kernel<false, true>), grid, block, 0, stream, a);
    else if (!a.b_kn) hipLaunchKernelGGL((gemm_bf16_kernel<true, false>), grid, block, 0, stream, a);
    else hipLaunchKernelGGL((gemm_bf16_kernel<true, true>), grid, block, 0, stream, a);
    if (a.ksplit > 1) {
        const size_t groups = ((size_t)a.M * a.N + 3) / 4;
        const unsigned sb = (unsigned)((groups + kThreads - 1) / kThreads < 4096 ? (groups + kThreads - 1) / kThreads : 4096);
        hipLaunchKernelGGL(gemm_splitk_sum_kernel, dim3(sb), dim3(kThreads), 0, stream, a);
    }
    return hipGetLastError();
}

}  // namespace cgqa
