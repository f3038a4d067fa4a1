// Device-side building blocks for the gfx950 attention kernels: vector types, the
// bf16 matrix-core instruction, the transposing LDS read and small lane helpers.
//
// Lane maps of v_mfma_f32_32x32x16_bf16 (wave64), as measured on gfx950:
//   A (32 x 16): lane l holds row m = l % 32, eight k slots of group h = l / 32.
//   B (16 x 32): lane l holds column n = l % 32, eight k slots of group h = l / 32.
//   A slot (h, s) multiplies B slot (h, s): which k a slot stands for is the
//   caller's choice, as long as A and B agree.
//   C (32 x 32): lane l register i holds row 8*(i/4) + 4*h + i%4, column n.
// ds_read_b64_tr_b16 works on groups of 16 lanes: if lane j of a group points at
// row j/4, columns 4*(j%4)..+3 of a 4 x 16 bf16 block, lane i of the group receives
// column i, rows 0..3. That is a column read of a row-major tile, which is how a
// matrix stored [k][n] becomes an MFMA operand whose slots run along k.
#pragma once
#include <hip/hip_runtime.h>

#include <type_traits>
#include <stdint.h>

namespace cgqa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint16_t u16x4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));

typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
typedef __fp16 fp16x4_raw __attribute__((__vector_size__(4 * sizeof(__fp16))));
typedef __attribute__((address_space(3))) fp16x4_raw lds_f16x4;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ f32x16 mfma32x32x16(const bf16x8& a, const bf16x8& b, const f32x16& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// The fp16 variant has the same lane maps.
__device__ __forceinline__ f32x16 mfma32x32x16(const f16x8& a, const f16x8& b, const f32x16& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 zero16() {
    f32x16 z;
#pragma unroll
    for (int i = 0; i < 16; ++i) z[i] = 0.0f;
    return z;
}

// 16-byte LDS read of eight bf16 (an A or B operand whose slots run along a row).
__device__ __forceinline__ bf16x8 lds_read8(const char* p) {
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(p));
}

// Transposing LDS read: see the lane map above. `p` is this lane's source address.
__device__ __forceinline__ bf16x4 lds_read_tr4(const char* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p));
}

__device__ __forceinline__ f16x8 lds_read8_f16(const char* p) {
    return __builtin_bit_cast(f16x8, *reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ f16x4 lds_read_tr4_f16(const char* p) {
    return __builtin_bit_cast(f16x4, __builtin_amdgcn_ds_read_tr16_b64_v4f16((lds_f16x4*)(p)));
}

__device__ __forceinline__ bf16x8 concat(const bf16x4& lo, const bf16x4& hi) {
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}
__device__ __forceinline__ f16x8 concat(const f16x4& lo, const f16x4& hi) {
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Eight bf16 values (as loaded, two per 32-bit word, the first in the low half) to
// fp16. bf16 -> fp32 is exact (the bf16 pattern is the upper half of the fp32 one);
// fp32 -> fp16 (v_cvt_pk_f16_f32, round to nearest even) is exact for magnitudes in
// [2^-14, 65504], since a bf16 value has only 8 significant bits.
__device__ __forceinline__ f16x8 bf16x8_to_f16(const u32x4& w) {
    f32x8 f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f[2 * i] = __builtin_bit_cast(float, w[i] << 16);
        f[2 * i + 1] = __builtin_bit_cast(float, w[i] & 0xFFFF0000u);
    }
    return __builtin_convertvector(f, f16x8);
}
__device__ __forceinline__ u32x4 bf16x8_to_f16_bits(const u32x4& w) {
    return __builtin_bit_cast(u32x4, bf16x8_to_f16(w));
}
// The same values times a power of two `s` (exact in fp32) before the fp16 rounding,
// one pair at a time (two fp32 temporaries live at once).
__device__ __forceinline__ u32x4 bf16x8_to_f16_bits_scaled(const u32x4& w, float s) {
    u32x4 out;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const f32x2 f = {__builtin_bit_cast(float, w[i] << 16) * s, __builtin_bit_cast(float, w[i] & 0xFFFF0000u) * s};
        out[i] = __builtin_bit_cast(uint32_t, __builtin_convertvector(f, f16x2));
    }
    return out;
}

// Eight accumulator registers (base .. base+7) rounded to bf16 (round to nearest
// even, v_cvt_pk_bf16_f32), in register order.
__device__ __forceinline__ bf16x8 pack_lo(const f32x16& c) {
    return __builtin_convertvector(c.lo, bf16x8);
}
__device__ __forceinline__ bf16x8 pack_hi(const f32x16& c) {
    return __builtin_convertvector(c.hi, bf16x8);
}
// The same, rounded to fp16 (round to nearest even).
__device__ __forceinline__ f16x8 pack_lo_f16(const f32x16& c) {
    return __builtin_convertvector(c.lo, f16x8);
}
__device__ __forceinline__ f16x8 pack_hi_f16(const f32x16& c) {
    return __builtin_convertvector(c.hi, f16x8);
}

// The largest magnitude among eight bf16 values (as loaded, two per 32-bit word), as its
// bit pattern without the sign: for finite values the bit patterns order like the
// magnitudes.
__device__ __forceinline__ unsigned bf16x8_absmax_bits(const u32x4& w) {
    u16x2 m = __builtin_bit_cast(u16x2, w[0] & 0x7FFF7FFFu);
#pragma unroll
    for (int i = 1; i < 4; ++i) m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2, w[i] & 0x7FFF7FFFu));
    return max((unsigned)m[0], (unsigned)m[1]);
}

// Largest value over the wave, on every lane: DPP swaps within quads, then the two
// mirrors fold each row of 16 lanes; the four row maxima are read as scalars.
__device__ __forceinline__ unsigned wave_max_u32(unsigned v) {
    v = max(v, (unsigned)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false));   // quad_perm 1,0,3,2
    v = max(v, (unsigned)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false));   // quad_perm 2,3,0,1
    v = max(v, (unsigned)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, false));  // row_half_mirror
    v = max(v, (unsigned)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xF, 0xF, false));  // row_mirror
    const unsigned r0 = (unsigned)__builtin_amdgcn_readlane((int)v, 0), r1 = (unsigned)__builtin_amdgcn_readlane((int)v, 16);
    const unsigned r2 = (unsigned)__builtin_amdgcn_readlane((int)v, 32), r3 = (unsigned)__builtin_amdgcn_readlane((int)v, 48);
    return max(max(r0, r1), max(r2, r3));
}

// An exact power-of-two scale that brings a value whose largest bf16 magnitude has the bit
// pattern `bits` into [1, 2), and its inverse: 2^(127 - E) and 2^(E - 127) for the value's
// exponent field E, clamped to [1, 253] so that both are normal fp32 numbers (a zero or
// subnormal maximum takes the largest scale). Multiplying by either is exact, and fp16
// rounding commutes with it wherever the values stay in fp16's normal range.
struct Pow2Scale {
    float s, inv;
};
__device__ __forceinline__ Pow2Scale pow2_normalizer(unsigned bits) {
    const int e = min(max((int)(bits >> 7), 1), 253);
    return {__uint_as_float((unsigned)(254 - e) << 23), __uint_as_float((unsigned)e << 23)};
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float log2_fast(float x) { return __builtin_amdgcn_logf(x); }

// Value held by the lane 32 positions away (the other k-group of the same column).
__device__ __forceinline__ float swap_halves(float x) { return __shfl_xor(x, 32, 64); }

// x of lane l combined with x of lane l ^ 32 through v_permlane32_swap (no LDS). Both
// lanes of a pair add (or compare) the low-half value first, so they get the same bits.
__device__ __forceinline__ float sum_halves(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float max_halves(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Kernel-local lambdas capture the kernel's register arrays by reference; they must be
// inlined, or those arrays would move to scratch memory.
#define CGQA_INLINE __attribute__((always_inline))

// Instruction-scheduling hints for a basic block (groups are filled in order).
constexpr int kSchedVALU = 0x002;
constexpr int kSchedMFMA = 0x008;
constexpr int kSchedDSRead = 0x100;
#define CGQA_SCHED_GROUP(mask, n) __builtin_amdgcn_sched_group_barrier((mask), (n), 0)

// True on every lane if `pred` holds on any active lane (a wave-uniform branch).
__device__ __forceinline__ bool wave_any(bool pred) { return __builtin_amdgcn_ballot_w64(pred) != 0; }

// Direct global -> LDS copy of 16 bytes per lane (global_load_lds_dwordx4): lane i's
// 16 bytes from `src` land at LDS byte address `lds_base + 16 * i` (M0 holds the
// base, which must be the same on every lane). Completion is counted by vmcnt like any
// vector memory load. The instruction is issued from inline asm so that the compiler
// does not treat every later LDS read as dependent on it (it would wait for all loads
// in flight, including the prefetch); callers order it with wait_tiles_barrier. For
// the compiler's own vmcnt bookkeeping the extra loads only make its waits longer,
// never shorter, since loads complete in order.
__device__ __forceinline__ void load_lds16(const uint16_t* src, const void* lds_base) {
    const unsigned m0 = __builtin_amdgcn_readfirstlane(
        (unsigned)(uintptr_t)(const __attribute__((address_space(3))) void*)lds_base);
    // M0 is reserved by the compiler, so the asm restores the value it found.
    unsigned saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %1, off\n\ts_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(src), "s"(m0)
        : "memory");
}

// As load_lds16, with the address split into a wave-uniform base (SGPR pair) and a
// per-lane 32-bit byte offset: one VGPR per lane instead of a 64-bit address pair.
__device__ __forceinline__ void load_lds16_off(const void* base, unsigned off, const void* lds_base) {
    const unsigned m0 = __builtin_amdgcn_readfirstlane(
        (unsigned)(uintptr_t)(const __attribute__((address_space(3))) void*)lds_base);
    // readfirstlane returns int: both halves are zero-extended through uint32_t (a
    // sign-extended low half would set every bit of the high word).
    const uint64_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((unsigned)(uintptr_t)base);
    const uint64_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((unsigned)((uintptr_t)base >> 32));
    const uint64_t sbase = lo | (hi << 32);
    unsigned saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %3\n\tglobal_load_lds_dwordx4 %1, %2\n\ts_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(off), "s"(sbase), "s"(m0)
        : "memory");
}

// N (1, 2 or 4) consecutive 1 KB chunks in one asm block, M0 saved and restored once.
// Chunk e lands at LDS byte address lds + 1024 * e + 16 * lane and reads global
// address base + off[e] + 1024 * e (the instruction offset applies to both), so
// callers pass off[e] already reduced by 1024 * e. base and lds are wave-uniform.
template <int N>
__device__ __forceinline__ void load_lds16_chunks(const void* base, const unsigned (&off)[N], unsigned lds) {
    static_assert(N == 1 || N == 2 || N == 4, "chunk count");
    const uint64_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((unsigned)(uintptr_t)base);
    const uint64_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((unsigned)((uintptr_t)base >> 32));
    const uint64_t sbase = lo | (hi << 32);
    const unsigned m0 = __builtin_amdgcn_readfirstlane(lds);
    unsigned saved;
    if constexpr (N == 1) {
        asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %1, %3\n\ts_mov_b32 m0, %0"
                     : "=&s"(saved) : "v"(off[0]), "s"(m0), "s"(sbase) : "memory");
    } else if constexpr (N == 2) {
        asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %3\n\t"
                     "global_load_lds_dwordx4 %1, %4\n\tglobal_load_lds_dwordx4 %2, %4 offset:1024\n\t"
                     "s_mov_b32 m0, %0"
                     : "=&s"(saved) : "v"(off[0]), "v"(off[1]), "s"(m0), "s"(sbase) : "memory");
    } else {
        asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %5\n\t"
                     "global_load_lds_dwordx4 %1, %6\n\tglobal_load_lds_dwordx4 %2, %6 offset:1024\n\t"
                     "global_load_lds_dwordx4 %3, %6 offset:2048\n\tglobal_load_lds_dwordx4 %4, %6 offset:3072\n\t"
                     "s_mov_b32 m0, %0"
                     : "=&s"(saved) : "v"(off[0]), "v"(off[1]), "v"(off[2]), "v"(off[3]), "s"(m0), "s"(sbase)
                     : "memory");
    }
}

// The 4-byte variant (global_load_lds_dword): lane i's 4 bytes land at lds_base + 4 * i.
__device__ __forceinline__ void load_lds4(const void* src, const void* lds_base) {
    const unsigned m0 = __builtin_amdgcn_readfirstlane(
        (unsigned)(uintptr_t)(const __attribute__((address_space(3))) void*)lds_base);
    unsigned saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\tglobal_load_lds_dword %1, off\n\ts_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(src), "s"(m0)
        : "memory");
}

// load_lds4 with the address split into a wave-uniform base and a 32-bit lane offset
// (bytes); lds is the wave-uniform LDS byte address.
__device__ __forceinline__ void load_lds4_off(const void* base, unsigned off, unsigned lds) {
    const uint64_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((unsigned)(uintptr_t)base);
    const uint64_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((unsigned)((uintptr_t)base >> 32));
    const uint64_t sbase = lo | (hi << 32);
    const unsigned m0 = __builtin_amdgcn_readfirstlane(lds);
    unsigned saved;
    asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\tglobal_load_lds_dword %1, %3\n\ts_mov_b32 m0, %0"
                 : "=&s"(saved) : "v"(off), "s"(m0), "s"(sbase) : "memory");
}

// Physical 16-byte slot of logical chunk c in LDS row r is c ^ chunk_swizzle<D>(r) for
// tiles written by direct-to-LDS loads (whose rows cannot be padded). LDS serves 64
// banks x 4 bytes per clock: a D=64 row (128 B) is half a bank window, a D=128 row a
// whole one. For 16 lanes reading the same chunk of 16 consecutive rows (an A operand)
// every (row parity, slot) pair, resp. slot, must differ; for a transposing read (4
// consecutive rows, an aligned pair of chunks) the slot pairs of rows that share a bank
// window must differ. Both hold for these maps.
template <int D>
__device__ __forceinline__ int chunk_swizzle(int r) {
    if constexpr (D == 64) {
        const int u = (r >> 1) & 7;
        return ((u & 1) << 2) | (((u >> 2) & 1) << 1) | ((u >> 1) & 1);
    } else {
        return ((r & 7) << 1) | ((r >> 3) & 1);
    }
}

// Kernel arguments sit in memory that the runtime may place on the host side of the bus
// (on some systems it does: every kernel then starts with a bus round trip). The compiler
// loads each argument where it is first needed and reloads it when it runs short of
// scalar registers, so a kernel can pay several such round trips, some of them late (in
// its epilogue). An opaque copy of every 32-bit word at kernel entry issues all the
// loads together and keeps the values in scalar registers from then on.
template <typename T>
__device__ __forceinline__ void pin_args(T& v) {
    static_assert(sizeof(T) % 4 == 0, "32-bit words");
    unsigned w[sizeof(T) / 4];
    __builtin_memcpy(w, &v, sizeof(T));
#pragma unroll
    for (unsigned i = 0; i < sizeof(T) / 4; ++i) asm volatile("" : "+s"(w[i]));
    __builtin_memcpy(&v, w, sizeof(T));
}

// Calls f(integral_constant<int, 0>) .. f(integral_constant<int, N-1>) in order: an
// unrolled loop whose index is a compile-time constant in the body.
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
    if constexpr (N > 0) {
        static_for<N - 1>(f);
        f(std::integral_constant<int, N - 1>{});
    }
}

// Wait until at most N vector memory operations of this wave are outstanding and all
// its LDS operations are done, then join the workgroup barrier. Unlike
// __syncthreads() it leaves the newer (prefetch) loads in flight. The asm is also a
// compiler memory barrier.
template <int N>
__device__ __forceinline__ void wait_tiles_barrier() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

// Wait until at most N vector memory operations of this wave are outstanding (no
// barrier, LDS operations not waited for).
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Workgroup barrier for LDS traffic only: waits for this wave's LDS operations, not for
// its global loads and stores (which __syncthreads() would drain too), then joins the
// barrier. Enough when the barrier only orders LDS writes before LDS reads.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Rotary embedding, forward: eight consecutive bf16 dims (four interleaved pairs, as
// loaded) turned by the cosines c and sines s of their pairs, y0 = x0 c - x1 s and
// y1 = x0 s + x1 c, each rounded to bf16 (nearest even) from the exact value.
// A bf16 input times an fp32 table value has at most 32 significant bits, so it is exact
// in fp64, and fma(x0, c, -(x1 s)) in fp64 rounds the exact y a single time, to 53 bits.
// Rounding that to fp32 and then to bf16 can only go wrong where the fp32 value lands
// exactly on a bf16 tie (low 16 bits 0x8000); there the fp64 value says on which side of
// the tie y lies, and the fp32 value is moved one unit that way before its rounding to
// bf16. The one case left is an exact y within 2^-53 of a tie without being one (bits 10
// to 53 of its significand all equal), which fp64 cannot resolve.
__device__ __forceinline__ float rope_bf16_ready(double y) {
    const float f = (float)y;
    unsigned u = __float_as_uint(f);
    if ((u & 0xFFFFu) == 0x8000u) {
        const double fd = (double)f;
        if (y != fd) u = ((y > fd) == (f > 0.0f)) ? u + 1u : u - 1u;
    }
    return __uint_as_float(u);
}
__device__ __forceinline__ u32x4 rope_turn8(u32x4 raw, f32x4 c, f32x4 s) {
    const bf16x8 x = __builtin_bit_cast(bf16x8, raw);
    f32x4 lo, hi;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const double x0 = (double)(float)x[2 * p], x1 = (double)(float)x[2 * p + 1];
        const double cp = (double)c[p], sp = (double)s[p];
        const double y0 = fma(x0, cp, -(x1 * sp));
        const double y1 = fma(x0, sp, x1 * cp);
        if (p < 2) { lo[2 * p] = rope_bf16_ready(y0); lo[2 * p + 1] = rope_bf16_ready(y1); }
        else { hi[2 * p - 4] = rope_bf16_ready(y0); hi[2 * p - 3] = rope_bf16_ready(y1); }
    }
    const u32x2 wlo = __builtin_bit_cast(u32x2, __builtin_convertvector(lo, bf16x4));
    const u32x2 whi = __builtin_bit_cast(u32x2, __builtin_convertvector(hi, bf16x4));
    u32x4 y;
    y[0] = wlo[0]; y[1] = wlo[1]; y[2] = whi[0]; y[3] = whi[1];
    return y;
}

// Rotary embedding, backward. The cosines and sines of the two pairs that start at dim
// `dim` (a multiple of 4) of position t, from [T][half_d] tables (8-byte aligned reads).
struct RopeCS {
    float2 c, s;
};
__device__ __forceinline__ RopeCS rope_load(const float* cos, const float* sin, size_t t, int half_d, int dim) {
    const size_t i = t * (size_t)half_d + (size_t)(dim / 2);
    return {*reinterpret_cast<const float2*>(cos + i), *reinterpret_cast<const float2*>(sin + i)};
}
// Four consecutive dims hold two pairs (x0, x1), (x2, x3) of a gradient with respect to
// rotated values; returns the gradient with respect to the unrotated ones, R^T x.
__device__ __forceinline__ f32x4 rope_back4(f32x4 x, RopeCS r) {
    f32x4 y;
    y[0] = fmaf(x[0], r.c.x, x[1] * r.s.x);
    y[1] = fmaf(x[1], r.c.x, -(x[0] * r.s.x));
    y[2] = fmaf(x[2], r.c.y, x[3] * r.s.y);
    y[3] = fmaf(x[3], r.c.y, -(x[2] * r.s.y));
    return y;
}

// Four consecutive outputs at element offset `off` of an output tensor that is fp32, or
// bf16 (rounded to nearest even) when `bf16` is set.
__device__ __forceinline__ void store_out4(void* base, size_t off, f32x4 x, bool bf16) {
    if (bf16)
        *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(base) + off) =
            __builtin_bit_cast(u32x2, __builtin_convertvector(x, bf16x4));
    else
        *reinterpret_cast<f32x4*>(static_cast<float*>(base) + off) = x;
}

__device__ __forceinline__ u32x4 load16(const uint16_t* p) {
    return *reinterpret_cast<const u32x4*>(p);
}
__device__ __forceinline__ void store16(char* p, const u32x4& v) {
    *reinterpret_cast<u32x4*>(p) = v;
}

}  // namespace cgqa
