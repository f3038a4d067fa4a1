// Naive causal grouped-query attention (page "A transformer in PTX", sections "Three
// ways to run it" and "Flash attention": the naive kernels write the whole T x T score
// matrix of every head to memory, and the fast kernels are checked against them on the
// GPU). Every step is its plain definition in fp32: scores, then a row softmax, then
// the products, each in a fixed summation order, with the probabilities kept in a
// caller-provided workspace of B*Hq*T*T floats. Only entries with key j <= query i are
// written or read.
//
//   forward:  S = scale * Q K^T;  P = softmax(S) over keys 0..i;  LSE = m + ln(sum);
//             O = P V (rounded to bf16, nearest even)
//   backward: P as above; dV = sum over the group's heads of P^T dO;
//             dP = dO V^T;  D_i = sum_j P_ij dP_ij;  dS = P (dP - D) (in place of P);
//             dQ = scale * dS K;  dK = scale * sum over the group's heads of dS^T Q
//
// Nothing here is tuned: tiles of 32 queries by 32 keys staged in LDS, one workgroup
// per row for the softmax, grid-stride loops over 64-bit tile counters.
#include "cgqa_launch.hpp"

namespace cgqa {
namespace {

constexpr int kNT = 32;          // queries (or keys) per tile
constexpr int kThreads = 256;
constexpr int kMaxD = 128;

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t x) { return __uint_as_float((uint32_t)x << 16); }

// Round to nearest even (finite inputs; a NaN stays a NaN).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
    const uint32_t u = __float_as_uint(f);
    if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu) != 0) return (uint16_t)((u >> 16) | 0x40u);
    return (uint16_t)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}

__device__ __forceinline__ size_t tok(int b, int T, int t) { return (size_t)b * T + t; }

// Workspace element (bh, i, j) of the [B*Hq][T][T] matrix.
__device__ __forceinline__ size_t pidx(int bh, int T, int i, int j) {
    return ((size_t)bh * T + i) * (size_t)T + j;
}

// Block-wide reduction over 256 threads in a fixed tree order (repeatable bits).
template <bool MAX>
__device__ float block_reduce(float x, float* red) {
    const int tid = threadIdx.x;
    red[tid] = x;
    __syncthreads();
    for (int s = kThreads / 2; s > 0; s >>= 1) {
        if (tid < s) red[tid] = MAX ? fmaxf(red[tid], red[tid + s]) : red[tid] + red[tid + s];
        __syncthreads();
    }
    const float r = red[0];
    __syncthreads();
    return r;
}

// S[bh, i, j] = scale * sum_c q[b, i, h, c] k[b, j, g, c] for j <= i, tile by tile.
__global__ __launch_bounds__(kThreads) void naive_scores_kernel(NaiveArgs a) {
    __shared__ float qs[kNT][kMaxD + 1];
    __shared__ float ks[kNT][kMaxD + 1];
    const int T = a.T, d = a.d, G = a.Hq / a.Hkv;
    const long nt = (T + kNT - 1) / kNT;
    const long total = (long)a.B * a.Hq * nt * nt;
    const int tx = threadIdx.x % kNT, ty = threadIdx.x / kNT;   // key column, group of 4 queries
    for (long tile = blockIdx.x; tile < total; tile += gridDim.x) {
        const int tj = (int)(tile % nt), ti = (int)(tile / nt % nt), bh = (int)(tile / (nt * nt));
        if (tj > ti) continue;   // every key of the tile is after every query: masked
        const int b = bh / a.Hq, h = bh % a.Hq, g = h / G;
        for (int e = threadIdx.x; e < kNT * d; e += kThreads) {
            const int r = e / d, c = e % d;
            const int i = ti * kNT + r, j = tj * kNT + r;
            qs[r][c] = i < T ? bf16_bits_to_f32(a.q[(tok(b, T, i) * a.Hq + h) * d + c]) : 0.0f;
            ks[r][c] = j < T ? bf16_bits_to_f32(a.k[(tok(b, T, j) * a.Hkv + g) * d + c]) : 0.0f;
        }
        __syncthreads();
        const int j = tj * kNT + tx;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int il = 4 * ty + r, i = ti * kNT + il;
            if (i < T && j <= i) {
                float acc = 0.0f;
                for (int c = 0; c < d; ++c) acc = fmaf(qs[il][c], ks[tx][c], acc);
                a.p[pidx(bh, T, i, j)] = a.scale * acc;
            }
        }
        __syncthreads();
    }
}

// Row (bh, i): m = max_j S, l = sum_j exp(S - m), P = exp(S - m) / l in place,
// lse = m + ln l.
__global__ __launch_bounds__(kThreads) void naive_softmax_kernel(NaiveArgs a) {
    __shared__ float red[kThreads];
    const int T = a.T;
    const long rows = (long)a.B * a.Hq * T;
    for (long r = blockIdx.x; r < rows; r += gridDim.x) {
        const int i = (int)(r % T), bh = (int)(r / T);
        float* row = a.p + pidx(bh, T, i, 0);
        float m = -INFINITY;
        for (int j = threadIdx.x; j <= i; j += kThreads) m = fmaxf(m, row[j]);
        m = block_reduce<true>(m, red);
        float l = 0.0f;
        for (int j = threadIdx.x; j <= i; j += kThreads) l += expf(row[j] - m);
        l = block_reduce<false>(l, red);
        const float inv = 1.0f / l;
        for (int j = threadIdx.x; j <= i; j += kThreads) row[j] = expf(row[j] - m) * inv;
        if (threadIdx.x == 0 && a.lse) a.lse[r] = m + logf(l);
    }
}

// Query-side product for rows of one (batch, query head): out[b, i, h, c] =
// mult * sum_{j <= i} W[bh, i, j] x[b, j, g, c] with W the workspace and x = v (O, bf16
// output) or k (dQ, fp32 output). Thread (row tid / 8, columns tid % 8 + 8u).
template <bool TO_BF16>
__global__ __launch_bounds__(kThreads) void naive_rows_kernel(NaiveArgs a, const uint16_t* x, void* out, float mult) {
    __shared__ float ws[kNT][kNT + 1];
    __shared__ float xs[kNT][kMaxD + 1];
    const int T = a.T, d = a.d, G = a.Hq / a.Hkv;
    const long nt = (T + kNT - 1) / kNT;
    const long total = (long)a.B * a.Hq * nt;
    const int il = threadIdx.x / 8, c0 = threadIdx.x % 8;
    for (long tile = blockIdx.x; tile < total; tile += gridDim.x) {
        const int ti = (int)(tile % nt), bh = (int)(tile / nt);
        const int b = bh / a.Hq, h = bh % a.Hq, g = h / G;
        const int i = ti * kNT + il;
        float acc[kMaxD / 8];
#pragma unroll
        for (int u = 0; u < kMaxD / 8; ++u) acc[u] = 0.0f;
        for (int tj = 0; tj <= ti; ++tj) {
            for (int e = threadIdx.x; e < kNT * kNT; e += kThreads) {
                const int r = e / kNT, jl = e % kNT;
                const int ii = ti * kNT + r, jj = tj * kNT + jl;
                ws[r][jl] = (ii < T && jj <= ii) ? a.p[pidx(bh, T, ii, jj)] : 0.0f;
            }
            for (int e = threadIdx.x; e < kNT * d; e += kThreads) {
                const int r = e / d, c = e % d, jj = tj * kNT + r;
                xs[r][c] = jj < T ? bf16_bits_to_f32(x[(tok(b, T, jj) * a.Hkv + g) * d + c]) : 0.0f;
            }
            __syncthreads();
#pragma unroll
            for (int u = 0; u < kMaxD / 8; ++u) {
                const int c = c0 + 8 * u;
                if (c < d)
                    for (int jl = 0; jl < kNT; ++jl) acc[u] = fmaf(ws[il][jl], xs[jl][c], acc[u]);
            }
            __syncthreads();
        }
        if (i < T) {
            const size_t o = (tok(b, T, i) * a.Hq + h) * d;
#pragma unroll
            for (int u = 0; u < kMaxD / 8; ++u) {
                const int c = c0 + 8 * u;
                if (c >= d) continue;
                if (TO_BF16) static_cast<uint16_t*>(out)[o + c] = f32_to_bf16_rne(mult * acc[u]);
                else static_cast<float*>(out)[o + c] = mult * acc[u];
            }
        }
    }
}

// Key-side product for the keys of one (batch, kv head): out[b, j, g, c] =
// mult * sum over the group's heads h (ascending) of sum_{i >= j} W[bh, i, j] x[b, i, h, c]
// with x = dO (dV) or q (dK); fp32 output. Thread (key tid / 8, columns tid % 8 + 8u).
__global__ __launch_bounds__(kThreads) void naive_cols_kernel(NaiveArgs a, const uint16_t* x, float* out, float mult) {
    __shared__ float ws[kNT][kNT + 1];   // [key][query]
    __shared__ float xs[kNT][kMaxD + 1];
    const int T = a.T, d = a.d, G = a.Hq / a.Hkv;
    const long nt = (T + kNT - 1) / kNT;
    const long total = (long)a.B * a.Hkv * nt;
    const int jl = threadIdx.x / 8, c0 = threadIdx.x % 8;
    for (long tile = blockIdx.x; tile < total; tile += gridDim.x) {
        const int tj = (int)(tile % nt), bg = (int)(tile / nt);
        const int b = bg / a.Hkv, g = bg % a.Hkv;
        const int j = tj * kNT + jl;
        float acc[kMaxD / 8];
#pragma unroll
        for (int u = 0; u < kMaxD / 8; ++u) acc[u] = 0.0f;
        for (int h = g * G; h < (g + 1) * G; ++h) {
            const int bh = b * a.Hq + h;
            for (int ti = tj; ti < nt; ++ti) {
                for (int e = threadIdx.x; e < kNT * kNT; e += kThreads) {
                    const int r = e / kNT, ql = e % kNT;   // key r, query ql
                    const int jj = tj * kNT + r, ii = ti * kNT + ql;
                    ws[r][ql] = (ii < T && jj <= ii) ? a.p[pidx(bh, T, ii, jj)] : 0.0f;
                }
                for (int e = threadIdx.x; e < kNT * d; e += kThreads) {
                    const int r = e / d, c = e % d, ii = ti * kNT + r;
                    xs[r][c] = ii < T ? bf16_bits_to_f32(x[(tok(b, T, ii) * a.Hq + h) * d + c]) : 0.0f;
                }
                __syncthreads();
#pragma unroll
                for (int u = 0; u < kMaxD / 8; ++u) {
                    const int c = c0 + 8 * u;
                    if (c < d)
                        for (int ql = 0; ql < kNT; ++ql) acc[u] = fmaf(ws[jl][ql], xs[ql][c], acc[u]);
                }
                __syncthreads();
            }
        }
        if (j < T) {
            const size_t o = (tok(b, T, j) * a.Hkv + g) * d;
#pragma unroll
            for (int u = 0; u < kMaxD / 8; ++u) {
                const int c = c0 + 8 * u;
                if (c < d) out[o + c] = mult * acc[u];
            }
        }
    }
}

// Query tile (bh, ti), key tiles tj = 0 .. ti: dP_ij = sum_c dO[b, i, h, c] v[b, j, g, c];
// D_i = sum_j P_ij dP_ij; then dS_ij = P_ij (dP_ij - D_i) in place of P and delta = D.
// dP is computed twice, in the same order, so both passes see the same bits. D sums
// each thread's keys (ascending tiles) and then the 32 key columns in order.
__global__ __launch_bounds__(kThreads) void naive_ds_kernel(NaiveArgs a) {
    __shared__ float os[kNT][kMaxD + 1];
    __shared__ float vs[kNT][kMaxD + 1];
    __shared__ float red[kNT][kNT + 1];
    __shared__ float dsum[kNT];
    const int T = a.T, d = a.d, G = a.Hq / a.Hkv;
    const long nt = (T + kNT - 1) / kNT;
    const long total = (long)a.B * a.Hq * nt;
    const int tx = threadIdx.x % kNT, ty = threadIdx.x / kNT;   // key column, group of 4 queries
    for (long tile = blockIdx.x; tile < total; tile += gridDim.x) {
        const int ti = (int)(tile % nt), bh = (int)(tile / nt);
        const int b = bh / a.Hq, h = bh % a.Hq, g = h / G;
        for (int e = threadIdx.x; e < kNT * d; e += kThreads) {
            const int r = e / d, c = e % d, i = ti * kNT + r;
            os[r][c] = i < T ? bf16_bits_to_f32(a.dO[(tok(b, T, i) * a.Hq + h) * d + c]) : 0.0f;
        }
        auto load_v = [&](int tj) {
            for (int e = threadIdx.x; e < kNT * d; e += kThreads) {
                const int r = e / d, c = e % d, j = tj * kNT + r;
                vs[r][c] = j < T ? bf16_bits_to_f32(a.v[(tok(b, T, j) * a.Hkv + g) * d + c]) : 0.0f;
            }
        };
        auto dp = [&](int il) {
            float acc = 0.0f;
            for (int c = 0; c < d; ++c) acc = fmaf(os[il][c], vs[tx][c], acc);
            return acc;
        };
        float part[4] = {0.0f, 0.0f, 0.0f, 0.0f};
        for (int tj = 0; tj <= ti; ++tj) {
            load_v(tj);
            __syncthreads();
            const int j = tj * kNT + tx;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int il = 4 * ty + r, i = ti * kNT + il;
                if (i < T && j <= i) part[r] = fmaf(a.p[pidx(bh, T, i, j)], dp(il), part[r]);
            }
            __syncthreads();
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) red[4 * ty + r][tx] = part[r];
        __syncthreads();
        if (threadIdx.x < kNT) {
            float D = 0.0f;
            for (int x = 0; x < kNT; ++x) D += red[threadIdx.x][x];
            dsum[threadIdx.x] = D;
            const int i = ti * kNT + threadIdx.x;
            if (i < T) a.delta[(size_t)bh * T + i] = D;
        }
        __syncthreads();
        for (int tj = 0; tj <= ti; ++tj) {
            load_v(tj);
            __syncthreads();
            const int j = tj * kNT + tx;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int il = 4 * ty + r, i = ti * kNT + il;
                if (i < T && j <= i) {
                    float* pij = a.p + pidx(bh, T, i, j);
                    *pij = *pij * (dp(il) - dsum[il]);
                }
            }
            __syncthreads();
        }
    }
}

unsigned grid_for(long work) { return (unsigned)(work < 65536 ? (work > 0 ? work : 1) : 65536); }

hipError_t scores_and_softmax(const NaiveArgs& a, hipStream_t stream) {
    const long nt = (a.T + kNT - 1) / kNT;
    hipLaunchKernelGGL(naive_scores_kernel, dim3(grid_for((long)a.B * a.Hq * nt * nt)), dim3(kThreads), 0, stream, a);
    hipLaunchKernelGGL(naive_softmax_kernel, dim3(grid_for((long)a.B * a.Hq * a.T)), dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_naive_fwd(const NaiveArgs& a, hipStream_t stream) {
    hipError_t e = scores_and_softmax(a, stream);
    if (e != hipSuccess) return e;
    const long nt = (a.T + kNT - 1) / kNT;
    hipLaunchKernelGGL((naive_rows_kernel<true>), dim3(grid_for((long)a.B * a.Hq * nt)), dim3(kThreads), 0, stream,
                       a, a.v, static_cast<void*>(a.o), 1.0f);
    return hipGetLastError();
}

hipError_t launch_naive_bwd(const NaiveArgs& a, hipStream_t stream) {
    hipError_t e = scores_and_softmax(a, stream);
    if (e != hipSuccess) return e;
    const long nt = (a.T + kNT - 1) / kNT;
    const unsigned gk = grid_for((long)a.B * a.Hkv * nt), gq = grid_for((long)a.B * a.Hq * nt);
    hipLaunchKernelGGL(naive_cols_kernel, dim3(gk), dim3(kThreads), 0, stream, a, a.dO, a.dv, 1.0f);
    hipLaunchKernelGGL(naive_ds_kernel, dim3(gq), dim3(kThreads), 0, stream, a);
    hipLaunchKernelGGL((naive_rows_kernel<false>), dim3(gq), dim3(kThreads), 0, stream, a, a.k,
                       static_cast<void*>(a.dq), a.scale);
    hipLaunchKernelGGL(naive_cols_kernel, dim3(gk), dim3(kThreads), 0, stream, a, a.q, a.dk, a.scale);
    return hipGetLastError();
}

}  // namespace cgqa
