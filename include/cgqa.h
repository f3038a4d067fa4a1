/*
 * cgqa: causal grouped-query flash attention for AMD MI355X (gfx950).
 *
 * The operation is the causal softmax attention of a Llama-style decoder with
 * grouped-query heads (page "A transformer in PTX", section "The model": groups of query
 * heads read one shared key/value head), computed as flash attention (section "Flash
 * attention": scores never go to memory; each row carries a running max and sum in
 * base-2 units; the forward stores each row's log-sum-exp so the backward can rebuild
 * the probabilities), with a deterministic two-kernel backward (section "The same bits
 * every time": one kernel owns blocks of queries and produces dQ, the other owns blocks
 * of keys and produces dK/dV, visiting every query head of the key/value head's group;
 * no float atomics, so repeated runs are bit-identical).
 *
 * Shapes and layout (all tensors contiguous, row-major, owned by the caller):
 *   q, o, dO : [B][T][Hq][d]   bfloat16 (passed as uint16_t bit patterns)
 *   k, v     : [B][T][Hkv][d]  bfloat16
 *   lse      : [B][Hq][T]      float32, natural-log log-sum-exp of each row of
 *                              scale * q.k over keys 0..i (causal, inclusive)
 *   delta    : [B][Hq][T]      float32, D_i = sum_j P_ij dP_ij (= sum_c dO[i,c] * O[i,c]
 *                              in exact arithmetic)
 *   dO_absmax: [B][Hq][NB]     float32, NB = ceil(T / 32): the largest |dO| over the 32
 *                              query rows 32*j .. 32*j+31 of head h (rows below T)
 *   dq       : [B][T][Hq][d]   float32
 *   dk, dv   : [B][T][Hkv][d]  float32
 * Query head h uses key/value head h / (Hq / Hkv). Query i sees keys 0..i.
 * d must be 64 or 128. Every pointer must be 16-byte aligned device memory.
 * The *_strided calls below take the same tensors with a row stride each (see there).
 *
 * Every call only enqueues work on `stream` (a hipStream_t; NULL = the default
 * stream) and returns; outputs are valid once the caller synchronises with the stream.
 * A fault while the kernels run surfaces at that synchronisation, not in the return
 * value. Calls allocate nothing, keep no state between calls and may be made from
 * several host threads at once. Outputs must not overlap inputs or each other.
 * B == 0 or T == 0 is an empty problem: the call succeeds and touches nothing.
 *
 * Numerics and value range. The forward's two products run on the bf16 matrix cores
 * with fp32 accumulation and an fp32 softmax. The backward's products that take the
 * probabilities P or dS = P (dP - D) run on the fp16 matrix cores with fp32
 * accumulation, so q, k and v are converted to fp16 there: their magnitudes must stay
 * below 65504 (beyond it gradients turn infinite), and values under 2^-14 keep fewer
 * significant bits than bf16 gives them. dO may have any bf16 magnitude, also one that
 * differs widely from row to row: before their fp16 rounding, dO and dS are scaled by
 * powers of two (per query row in attn_bwd_dq; in attn_bwd_dkv by one scale per batch and
 * key/value head, from the largest |dO| of the group's query heads, which attn_bwd_dq
 * publishes in dO_absmax) and the sums are scaled back in fp32. Multiplying dO by 2^k
 * therefore multiplies delta, dq, dk and dv by exactly 2^k, short of fp32 underflow or
 * overflow. dS stays finite whenever every row of v has sum_c |v_c| < 16000.
 *
 * Return value: CGQA_OK (0) or one of the codes below. All argument checks happen
 * before any HIP call, so a rejected call has touched neither the device nor the
 * stream.
 */
#ifndef CGQA_H
#define CGQA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
    CGQA_OK = 0,
    /* null pointer with non-empty sizes, negative size, Hq or Hkv < 1, Hq % Hkv != 0,
       scale not finite or not positive, an element count of 2^31 or more, a row stride
       shorter than its row, an unknown gradient type, or an output that overlaps
       another buffer */
    CGQA_EINVAL = 1,
    /* head dimension other than 64 or 128, a pointer not 16-byte aligned, or a row
       stride that is not a whole number of 16-byte units (inputs) or 8-byte units
       (outputs) */
    CGQA_EUNSUPPORTED = 2,
    /* the kernel launch was refused by the HIP runtime (cgqa_last_hip_error() tells
       which HIP error, for the calling thread) */
    CGQA_EHIP = 3
};

/* Forward (section "Flash attention"): o = softmax(scale * q k^T, causal) v per query
 * head, and lse = the natural-log log-sum-exp of each row of scaled scores.
 * Reads q, k, v; overwrites o and lse. */
int attn_fwd(const uint16_t* q, const uint16_t* k, const uint16_t* v,
             uint16_t* o, float* lse,
             int B, int T, int Hq, int Hkv, int d, float scale, void* stream);

/* Backward, query side (section "The same bits every time": each block of queries
 * has a single owning workgroup). For the loss L = sum(O * dO): recomputes P from q, k
 * and lse, writes delta = D_i = sum_j P_ij dP_ij (accumulated in fp32 inside the kernel;
 * it equals rowsum(dO * O), which the bf16 o would give only to bf16 accuracy),
 * dO_absmax (the caller-owned workspace that carries the scale of dO to attn_bwd_dkv,
 * B*Hq*ceil(T/32) floats) and dq = dL/dq. Reads q, k, v, o, dO, lse; overwrites delta,
 * dO_absmax and dq. */
int attn_bwd_dq(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                const uint16_t* o, const uint16_t* dO, const float* lse,
                float* delta, float* dO_absmax, float* dq,
                int B, int T, int Hq, int Hkv, int d, float scale, void* stream);

/* Backward, key side (same section: each block of keys has a single owning workgroup,
 * which visits the query heads of its key/value head's group in ascending order and,
 * for each, the query blocks in ascending order). Writes dk = dL/dk and dv = dL/dv, summed over the
 * group. Reads the delta and dO_absmax written by attn_bwd_dq for the same dO, so it
 * must be enqueued after that call on the same stream (or after an event recorded
 * behind it). Reads q, k, v, dO, lse, delta, dO_absmax; overwrites dk and dv. */
int attn_bwd_dkv(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                 const uint16_t* dO, const float* lse, const float* delta,
                 const float* dO_absmax, float* dk, float* dv,
                 int B, int T, int Hq, int Hkv, int d, float scale, void* stream);

/* Strided variants: the same operations on tensors that sit inside wider rows, e.g. the
 * packed [B*T][(Hq + 2*Hkv)*d] buffer that one fused projection produces for queries,
 * keys and values (page "A transformer in PTX", section "The model": one fused matmul
 * computes them) with q = base, k = base + Hq*d, v = base + (Hq + Hkv)*d, and gradients
 * written into a packed buffer of the same shape.
 *
 * Element (b, t, h, c) of a tensor with row stride rs is at (b*T + t)*rs + h*d + c, in
 * elements of the tensor's own type; rs = H*d is the contiguous layout of the calls
 * above, which these reproduce bit for bit. Each stride must be at least its row (H*d)
 * and at most such that B*T*rs < 2^31. The strides of bf16 tensors a call reads (q, k
 * and v; o and dO in the backward) must be multiples of 8 elements, those of the outputs
 * (o in the forward; dq, dk and dv) multiples of 4 elements.
 * k and v share kv_row_stride; dk and dv share dkv_row_stride.
 *
 * grad_dtype selects the type of dq, dk and dv: CGQA_GRAD_F32 (float) or CGQA_GRAD_BF16
 * (bfloat16 bit patterns, rounded to nearest even from the same float values the float
 * outputs hold). lse and delta stay [B][Hq][T] float32, dO_absmax [B][Hq][ceil(T/32)].
 *
 * Outputs may share a buffer with each other when their row strides (in bytes) are
 * equal and their column ranges within a row do not meet (dq, dk, dv of one packed
 * buffer); any other overlap of an output with another tensor is CGQA_EINVAL. */
enum { CGQA_GRAD_F32 = 0, CGQA_GRAD_BF16 = 1 };

int attn_fwd_strided(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                     uint16_t* o, float* lse,
                     int B, int T, int Hq, int Hkv, int d,
                     int q_row_stride, int kv_row_stride, int o_row_stride,
                     float scale, void* stream);

int attn_bwd_dq_strided(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                        const uint16_t* o, const uint16_t* dO, const float* lse,
                        float* delta, float* dO_absmax, void* dq,
                        int B, int T, int Hq, int Hkv, int d,
                        int q_row_stride, int kv_row_stride, int o_row_stride,
                        int do_row_stride, int dq_row_stride, int grad_dtype,
                        float scale, void* stream);

int attn_bwd_dkv_strided(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                         const uint16_t* dO, const float* lse, const float* delta,
                         const float* dO_absmax, void* dk, void* dv,
                         int B, int T, int Hq, int Hkv, int d,
                         int q_row_stride, int kv_row_stride, int do_row_stride,
                         int dkv_row_stride, int grad_dtype, float scale, void* stream);

/* Rotary position embedding around attention (page "A transformer in PTX", section "The
 * model": the fused QKV matmul's queries and keys are rotated with RoPE, in place in the
 * bf16 buffer, before causal attention). Pair i = (x[2i], x[2i+1]) of every head of token
 * t turns by the angle whose cosine and sine are cos[t][i] and sin[t][i] (caller tables,
 * fp32 [T][d/2], 16-byte aligned):
 *   y[2i] = x[2i] cos - x[2i+1] sin,   y[2i+1] = x[2i] sin + x[2i+1] cos.
 *
 * attn_rope_qk writes the rotated q and k as bf16, each value rounded to nearest (ties to
 * even) from the exact rotated value (computed with one fp64 rounding, which decides every
 * case but an exact value within 2^-53 relative of a bf16 tie without being one); tensors
 * are [B][T][H][d] with row strides as in the strided calls (multiples of 8). An output
 * may be its own input (same pointer and stride: in place, e.g. on the packed QKV buffer);
 * any other overlap of an output is CGQA_EINVAL. The forward then runs attn_fwd on the
 * rotated tensors.
 *
 * attn_fwd_rope is attn_fwd on q and k rotated as they are loaded, with no rotated copy
 * written: q and k are the unrotated contiguous tensors, and o and lse are those of
 * attention on the rotated ones, each rotated value rounded exactly as attn_rope_qk
 * rounds it (the same bits as attn_rope_qk followed by attn_fwd wherever attn_fwd runs
 * its tiled kernel, i.e. at least three 128-query workgroups per CU). d = 64 only
 * (CGQA_EUNSUPPORTED otherwise); missing tables are CGQA_EINVAL, tables not 16-byte
 * aligned CGQA_EUNSUPPORTED, tables overlapping o or lse CGQA_EINVAL. Every workgroup
 * that reads a K tile turns it again, so this call is slower than attn_rope_qk followed
 * by attn_fwd; it serves callers that keep no rotated copy of q and k. A backward on its
 * outputs needs the rotated tensors (attn_rope_qk) all the same.
 *
 * attn_bwd_dq_rope / attn_bwd_dkv_rope are attn_bwd_dq / attn_bwd_dkv on the rotated q and k
 * (contiguous, fp32 gradients) whose dq and dk are turned back inside the kernels, before
 * they are stored, to the gradients with respect to the unrotated q and k:
 *   g[2i] = gy[2i] cos + gy[2i+1] sin,   g[2i+1] = -gy[2i] sin + gy[2i+1] cos
 * (dv, delta and dO_absmax are unchanged). */
int attn_rope_qk(const uint16_t* q, const uint16_t* k, uint16_t* q_out, uint16_t* k_out,
                 const float* cos, const float* sin, int B, int T, int Hq, int Hkv, int d,
                 int q_row_stride, int k_row_stride, int q_out_row_stride, int k_out_row_stride,
                 void* stream);

int attn_fwd_rope(const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* o, float* lse,
                  const float* cos, const float* sin, int B, int T, int Hq, int Hkv, int d,
                  float scale, void* stream);

int attn_bwd_dq_rope(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                     const uint16_t* o, const uint16_t* dO, const float* lse,
                     float* delta, float* dO_absmax, float* dq, const float* cos, const float* sin,
                     int B, int T, int Hq, int Hkv, int d, float scale, void* stream);

int attn_bwd_dkv_rope(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                      const uint16_t* dO, const float* lse, const float* delta,
                      const float* dO_absmax, float* dk, float* dv, const float* cos, const float* sin,
                      int B, int T, int Hq, int Hkv, int d, float scale, void* stream);

/* Naive attention, the GPU reference mode (page "A transformer in PTX", section "Three
 * ways to run it": the fast kernels are checked against naive ones; section "Flash
 * attention": naive kernels store the whole T x T score matrix of every head). Same
 * operation, shapes and layouts as attn_fwd / attn_bwd_dq + attn_bwd_dkv for contiguous
 * tensors, computed step by step in fp32: scores into `workspace`, a row softmax in place,
 * then the products, each sum in a fixed order (repeatable bits). d may be any value from
 * 1 to 128 (CGQA_EUNSUPPORTED otherwise).
 *
 * workspace: caller-owned device memory of at least attn_naive_workspace_bytes(B, T, Hq)
 * bytes (fp32 [B][Hq][T][T]; only entries with key <= query are used), 16-byte aligned,
 * overlapping no other argument; its contents on return are unspecified. A missing or
 * smaller workspace is CGQA_EINVAL. Calls that share a workspace must be ordered on the
 * GPU (one stream, or events).
 *
 * attn_naive_fwd writes o (bf16, rounded to nearest even from fp32) and lse.
 * attn_naive_bwd recomputes the probabilities itself (it reads no o or lse) and writes
 * delta = D_i = sum_j P_ij dP_ij and the fp32 gradients dq, dk, dv of L = sum(O * dO). */
size_t attn_naive_workspace_bytes(int B, int T, int Hq);   /* 0 for sizes no call accepts */

int attn_naive_fwd(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                   uint16_t* o, float* lse, float* workspace, size_t workspace_bytes,
                   int B, int T, int Hq, int Hkv, int d, float scale, void* stream);

int attn_naive_bwd(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* dO,
                   float* delta, float* dq, float* dk, float* dv,
                   float* workspace, size_t workspace_bytes,
                   int B, int T, int Hq, int Hkv, int d, float scale, void* stream);

/* Matrix product of the projections around attention (page "A transformer in PTX",
 * section "Three ways to run it": one matmul kernel with layout flags, so dx = dy W and
 * dW = dy^T x run without transposing memory, and with an optional matrix added to the
 * product, e.g. the residual stream or a gradient accumulated across micro-batches):
 *
 *   C[m][n] = sum_k A[m][k] * B[n][k]  (+ R[m][n])
 *
 * A is bf16 [M][K] row-major, or [K][M] with CGQA_GEMM_A_KM; B is bf16 [N][K] (a weight
 * stored [out][in], as x W^T uses it), or [K][N] with CGQA_GEMM_B_KN. C is fp32 [M][N], or
 * bf16 with CGQA_GEMM_C_BF16 (rounded to nearest even). R is null or fp32 [M][N]; it may
 * be C itself when C is fp32 (C += A B^T), otherwise it must not overlap C. Products
 * accumulate in fp32 with k ascending; the bits of C do not depend on the layout flags.
 *
 * K must be a multiple of 32; with CGQA_GEMM_A_KM, M a multiple of 8; with CGQA_GEMM_B_KN,
 * N a multiple of 8 (CGQA_EUNSUPPORTED otherwise). M*K, N*K and M*N must stay below 2^31,
 * unknown flag bits are CGQA_EINVAL, and C must not overlap A or B. M == 0 or N == 0 is a
 * no-op; K == 0 writes C = R (or zeros) and then A and B may be null. Same stream,
 * alignment and error rules as above.
 *
 * workspace: null, or caller-owned fp32 device memory of workspace_bytes (16-byte aligned,
 * overlapping no other argument). Shapes with few 128 x 128 output tiles and a long K (a
 * weight gradient dW = dy^T x) then split K over several workgroups per tile that write
 * fp32 partial products there, summed afterwards in split order; at most
 * cgqa_gemm_workspace_bytes(M, N, K) bytes are used (0: this shape never splits). The
 * split count, and so the exact bits of C, depend only on M, N, K and workspace_bytes. */
enum { CGQA_GEMM_A_KM = 1, CGQA_GEMM_B_KN = 2, CGQA_GEMM_C_BF16 = 4 };

size_t cgqa_gemm_workspace_bytes(int M, int N, int K);

int cgqa_gemm(const uint16_t* A, const uint16_t* B, void* C, const float* R,
              int M, int N, int K, int flags, float* workspace, size_t workspace_bytes,
              void* stream);

/* For callers that cannot allocate: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc. cgqa_gemm_static is cgqa_gemm without a workspace
 * argument: a K split keeps its fp32 partials in a device array of
 * CGQA_GEMM_STATIC_SCRATCH_BYTES that the library holds on each GPU it runs on until the
 * process ends. C comes out bit for bit as from cgqa_gemm given a workspace of at least
 * cgqa_gemm_workspace_bytes(M, N, K) bytes. A shape whose split needs more than the array
 * holds (cgqa_gemm_workspace_bytes(M, N, K) > CGQA_GEMM_STATIC_SCRATCH_BYTES) is
 * CGQA_EINVAL, checked before any HIP call; the other argument rules are cgqa_gemm's. The
 * call allocates and frees nothing. Every call on one GPU shares that GPU's array, which
 * keeps the last call's partials (each split writes its whole slice before it is read,
 * so nothing needs clearing): calls that may overlap on one GPU, e.g. on two streams
 * with no ordering between them, race and give wrong results; order them. The first
 * call on a GPU looks the array's address up on that GPU (no allocation). */
#define CGQA_GEMM_STATIC_SCRATCH_BYTES ((size_t)16 << 20)

int cgqa_gemm_static(const uint16_t* A, const uint16_t* B, void* C, const float* R,
                     int M, int N, int K, int flags, void* stream);

/* Calibration, not attention: the rate the matrix core reaches on this GPU, so kernels can
 * be reported against a measured peak beside the spec sheet's (page "Talking to the GPU",
 * section "The real tensor core peak", times a kernel that only does tensor-core products).
 * Runs `blocks` workgroups of 256 threads; each wave issues 4 independent chains of `iters`
 * 32x32x16 bf16 matrix products on register operands (all 1/64) and each thread stores
 * iters / 64 (exact) to sink[block * 256 + thread] (device memory of blocks * 256 floats,
 * 16-byte aligned). clocks, if not null (device memory of 2 values, 16-byte aligned), gets
 * block 0's loop time as shader clocks and as ticks of the constant 100 MHz counter, whose
 * ratio is the clock the matrix cores ran at. *flops, if not null (host memory), receives
 * the flop count of the launch (2 flops per multiply-add); its time comes from the caller's
 * events. 1 <= blocks <= 65536, 1 <= iters <= 2^20, else CGQA_EINVAL. */
int cgqa_calib_mfma(float* sink, uint64_t* clocks, int blocks, int iters, double* flops, void* stream);

/* Static description of a return code (never NULL): every call reports failure as a code
 * whose meaning can be printed, the library-side form of the pages' practice of naming each
 * failed call and the error behind it (page "Talking to the GPU", section "One macro for
 * every call"; a library returns the code instead of exiting). */
const char* attn_status_string(int status);

/* The HIP error code behind the calling thread's last CGQA_EHIP (0 if none). */
int cgqa_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* CGQA_H */
