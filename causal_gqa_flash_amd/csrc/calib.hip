// Calibration, not attention: the rate the matrix core actually reaches on this chip,
// so that the attention kernels can be reported against a measured peak beside the
// spec sheet's (page "Talking to the GPU", section "The real tensor core peak": the
// pages time a kernel that does nothing but tensor-core products and report against
// that, with the clock it actually ran at). Every wave runs kChains independent chains of
// v_mfma_f32_32x32x16_bf16 on register operands, with no memory traffic until one store
// at the end; thread 0 of block 0 reads the shader clock counter and the constant
// 100 MHz real-time counter before and after its loop, whose ratio is the clock.
#include "cgqa_device.hpp"
#include "cgqa_launch.hpp"

namespace cgqa {
namespace {

constexpr int kChains = 4;

__global__ __launch_bounds__(kCalibThreads) void mfma_peak_kernel(float* sink, unsigned long long* clocks,
                                                                   int iters) {
    const bool timer = clocks && blockIdx.x == 0 && threadIdx.x == 0;
    unsigned long long t0 = 0, r0 = 0;
    if (timer) {
        t0 = __builtin_amdgcn_s_memtime();
        r0 = __builtin_amdgcn_s_memrealtime();
    }
    // Every operand is 1/64 (bf16 0x3C80): each product adds 16 * 2^-12 = 2^-8 to every
    // accumulator element, so after `iters` steps each holds iters / 256 exactly.
    bf16x8 a;
#pragma unroll
    for (int i = 0; i < 8; ++i) a[i] = __builtin_bit_cast(__bf16, (unsigned short)0x3C80u);
    f32x16 c[kChains];
#pragma unroll
    for (int j = 0; j < kChains; ++j) c[j] = zero16();
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int j = 0; j < kChains; ++j) c[j] = mfma32x32x16(a, a, c[j]);
    }
    float s = 0.0f;
#pragma unroll
    for (int j = 0; j < kChains; ++j) s += c[j][(5 * j) & 15];
    sink[(size_t)blockIdx.x * kCalibThreads + threadIdx.x] = s;
    if (timer) {
        const unsigned long long t1 = __builtin_amdgcn_s_memtime();
        const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
        clocks[0] = t1 - t0;      // shader clocks
        clocks[1] = r1 - r0;      // 100 MHz ticks
    }
}

}  // namespace

double calib_mfma_flops(int blocks, int iters) {
    return (double)blocks * (kCalibThreads / 64) * kChains * (double)iters * (2.0 * 32 * 32 * 16);
}

hipError_t launch_calib_mfma(float* sink, unsigned long long* clocks, int blocks, int iters, hipStream_t stream) {
    hipLaunchKernelGGL(mfma_peak_kernel, dim3((unsigned)blocks), dim3(kCalibThreads), 0, stream, sink, clocks, iters);
    return hipGetLastError();
}

}  // namespace cgqa
