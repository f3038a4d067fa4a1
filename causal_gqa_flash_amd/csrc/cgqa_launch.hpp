// Host-side launch interface between the C-ABI entry points and the kernels.
// Arguments arrive here already validated (shapes, alignment, d in {64, 128}).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace cgqa {

// Largest grid the forward launcher balances with an explicit task map: three rounds
// of workgroups on 256 CUs (all resident at once).
constexpr int kFwdMaxMapped = 768;

struct FwdArgs {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    uint16_t* o;
    float* lse;
    int B, T, Hq, Hkv, d;
    float scale_log2;   // scale * log2(e): scores in log2 units
    int n_qtiles;       // set by the launcher
    int use_map;        // set by the launcher: task of workgroup x is task_map[x]
    uint16_t task_map[kFwdMaxMapped];
};

struct BwdArgs {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    const uint16_t* o;
    const uint16_t* dO;
    const float* lse;
    float* delta;       // written by the dq kernel, read by the dkv kernel
    float* dq;
    float* dk;
    float* dv;
    int B, T, Hq, Hkv, d;
    float scale;        // softmax scale (dS carries it into dQ and dK)
    float scale_log2;   // scale * log2(e)
    int n_tiles;        // set by the launcher
    int zigzag;         // dK/dV: deal key blocks in zig-zag order (set by the launcher)
};

hipError_t launch_fwd(const FwdArgs& a, hipStream_t stream);
hipError_t launch_bwd_dq(const BwdArgs& a, hipStream_t stream);
hipError_t launch_bwd_dkv(const BwdArgs& a, hipStream_t stream);

}  // namespace cgqa
