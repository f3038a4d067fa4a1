// Host-side launch interface between the C-ABI entry points and the kernels.
// Arguments arrive here already validated (shapes, alignment, d in {64, 128}).
//
// Tensor layout: element (b, t, h, c) of a [B, T, H, d] tensor with row stride rs (elements
// between consecutive tokens, rs >= H*d) sits at (b*T + t)*rs + h*d + c; rs = H*d is the
// contiguous layout. LSE and delta are always [B, Hq, T].
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace cgqa {

struct FwdArgs {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    uint16_t* o;
    float* lse;
    int B, T, Hq, Hkv, d;
    int q_rs, kv_rs, o_rs;   // row strides of Q, of K and V, of O (elements)
    float scale_log2;   // scale * log2(e): scores in log2 units
    int n_qtiles;       // set by the launcher: query tiles per (batch, head)
    int n_pairs;        // set by the launcher: B * Hkv (batch, kv head) slices
    int xcd_group;      // set by the launcher: keep each slice's tiles on one XCD
};

struct BwdArgs {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    const uint16_t* o;
    const uint16_t* dO;
    const float* lse;
    float* delta;       // written by the dq kernel, read by the dkv kernel
    void* dq;           // fp32, or bf16 when grad_bf16
    void* dk;
    void* dv;
    int B, T, Hq, Hkv, d;
    int q_rs, kv_rs, o_rs, do_rs;   // input row strides (elements)
    int dq_rs, dkv_rs;              // output row strides (elements of the output type)
    int grad_bf16;                  // 1: dQ, dK, dV rounded to bf16 (nearest even)
    float scale;        // softmax scale (dS carries it into dQ and dK)
    float scale_log2;   // scale * log2(e)
    int n_tiles;        // set by the launcher
    int zigzag;         // dK/dV: deal key blocks in zig-zag order (set by the launcher)
};

// Naive attention (attn_naive.hip): contiguous tensors, fp32 workspace p of B*Hq*T*T
// floats, 1 <= d <= 128.
struct NaiveArgs {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    const uint16_t* dO;   // backward only
    uint16_t* o;          // forward only
    float* lse;           // forward only (null in the backward, which recomputes P)
    float* delta;         // backward only
    float* dq;
    float* dk;
    float* dv;
    float* p;             // workspace
    int B, T, Hq, Hkv, d;
    float scale;
};

hipError_t launch_fwd(const FwdArgs& a, hipStream_t stream);
// Balanced forward for d = 64 and whole 64-query blocks (attn_fwd_split.hip).
bool fwd_split_supported(const FwdArgs& a);
long fwd_split_blocks(const FwdArgs& a);
hipError_t launch_fwd_split(const FwdArgs& a, hipStream_t stream);
hipError_t launch_bwd_dq(const BwdArgs& a, hipStream_t stream);
hipError_t launch_bwd_dkv(const BwdArgs& a, hipStream_t stream);
hipError_t launch_naive_fwd(const NaiveArgs& a, hipStream_t stream);
hipError_t launch_naive_bwd(const NaiveArgs& a, hipStream_t stream);

}  // namespace cgqa
