/*
 * tri_attn.h — C ABI of the MI355X (gfx950) triangle-attention library.
 *
 * Operation (TurboPairFormer pages: Lambda post, section "Как работает
 * TurboPairFormer"; biocloudservice page, section "它优化了什么"):
 * Pairformer triangle attention around the starting node.  For batch b, row i
 * and head h, the queries q[b,i,j,h,:] attend over the keys k[b,i,k,h,:] of the
 * same row with
 *     s[j,k] = alpha * <q[b,i,j,h,:], k[b,i,k,h,:]> + bias[b,h,j,k] + mu[b,i,k]
 *     o[b,i,j,h,:] = sum_k softmax_k(s[j,:])[k] * v[b,i,k,h,:]
 * where alpha is the softmax scale and mu is 0 for an attended key and -inf
 * for a masked one.  The pair bias is shared by every row i, so its gradient
 * is a sum over all rows.  The backward returns the query, key, value and
 * pair-bias gradients.
 *
 * Ending node (TRI_ATTN_FLAG_ENDING_NODE): the same operation on the pair
 * tensor with its two pair axes swapped: row r is the second pair index, the
 * queries and keys run along the first.  q, k, v, o, dO and the gradients stay
 * in the caller's [B,N,N,H,D] layout and are read and written through swapped
 * strides; the mask is read as mask[b, k, r]; the bias is used as given.
 *
 * Layouts (row-major, last index fastest):
 *   q, k, v, o, d_o, dq, dk, dv : bf16 [B, N, N, H, D]  (D contiguous)
 *   o_residual                  : fp32 [B, N, N, H, D] (bf16 with FLAG_RESIDUAL_BF16)
 *   bias, dbias                 : bf16 [B, H, N, N] (dbias fp32 with FLAG_DBIAS_FP32);
 *                                 bias values must lie in the fp16 range
 *                                 (|bias| <= 65504, or -inf): the kernels hold the
 *                                 bias as fp16, to which such a bf16 value converts
 *                                 exactly when |bias| >= 2^-14 (smaller magnitudes
 *                                 round to a multiple of 2^-24)
 *   mask                        : uint8 [B, N, N], nonzero = key attended; NULL = all
 *   lse                         : fp32 [B, N, H, N], indexed [b, r, h, q] by
 *                                 attention row r and query q (natural log)
 *
 * Conventions shared by every entry point:
 *   - All tensor pointers are device pointers owned by the caller.  The library
 *     allocates nothing, frees nothing and keeps no pointer after returning.
 *   - Work is enqueued on `stream`; the call returns without synchronising.
 *   - Arguments are validated on the host before any HIP call.  On an error
 *     nothing is enqueued and no output is touched.  Unsupported sizes return
 *     TRI_ATTN_ERROR_NOT_SUPPORTED; there is no silent fallback path.
 *   - Tensor base pointers must be 16-byte aligned and outputs must not overlap
 *     inputs.
 *   - Results are bitwise deterministic for a fixed problem, build and device:
 *     every reduction runs in a fixed order and no floating-point atomics are
 *     used (Lambda post, "Как работает TurboPairFormer", third point).
 *   - No global mutable state: calls from several threads are safe.
 */
#ifndef TRI_ATTN_H
#define TRI_ATTN_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TRI_ATTN_ABI_VERSION 3

typedef enum {
    TRI_ATTN_SUCCESS = 0,
    TRI_ATTN_ERROR_INVALID_VALUE = 1,          /* null pointer, bad size, misalignment, aliasing */
    TRI_ATTN_ERROR_NOT_SUPPORTED = 2,          /* valid request this build does not implement */
    TRI_ATTN_ERROR_INSUFFICIENT_WORKSPACE = 3, /* workspace_bytes below tri_attn_bwd_workspace_bytes */
    TRI_ATTN_ERROR_LAUNCH_FAILED = 4,          /* a kernel launch reported an error */
    TRI_ATTN_ERROR_ABI_MISMATCH = 5            /* problem.abi_version != TRI_ATTN_ABI_VERSION */
} tri_attn_status;

enum {
    TRI_ATTN_FLAG_ENDING_NODE = 1 << 0,   /* attend along the first pair axis (see above) */
    TRI_ATTN_FLAG_DBIAS_FP32 = 1 << 1,    /* dbias is written as fp32 instead of bf16 */
    TRI_ATTN_FLAG_RESIDUAL_BF16 = 1 << 2  /* o_residual is stored as bf16 instead of fp32 (both passes) */
};

typedef struct {
    int32_t abi_version;  /* must equal TRI_ATTN_ABI_VERSION */
    int32_t flags;        /* TRI_ATTN_FLAG_* */
    int64_t B, N, H, D;   /* batch, pair length (I = J = K = N), heads, head dim */
    float softmax_scale;  /* alpha; 0 selects 1/sqrt(D) */
} tri_attn_problem;

/* Supported sizes of this build: D == 32 or D == 16, N a multiple of 32 with
 * 32 <= N <= 768, B >= 1, 1 <= H <= 64.  D == 16 runs the same kernels with the
 * tiles' channels 16..31 held at zero. */

/* Returns TRI_ATTN_ABI_VERSION of the loaded library. */
int tri_attn_abi_version(void);

/* Static, human-readable name of a status code (never NULL). */
const char *tri_attn_status_string(int status);

/*
 * Forward pass (Lambda post, "Как работает TurboPairFormer", second point:
 * the FP32-to-BF16 rounding residual of the output is kept for the backward).
 *   q, k, v, bias, mask : inputs as laid out above (mask may be NULL)
 *   o                   : bf16 output, round-to-nearest-even of the fp32 result O
 *   o_residual          : the fp32 residual O - float(o), exact in fp32, so that
 *                         float(o) + o_residual is O bitwise.  With
 *                         TRI_ATTN_FLAG_RESIDUAL_BF16 it is stored as its bf16
 *                         round-to-nearest-even instead (half the bytes): float(o)
 *                         + float(o_residual) then restores O to within 2^-9 of the
 *                         residual, about 2^-17 relative to O.  NULL = not saved
 *   lse                 : fp32 log-sum-exp of every softmax row; +inf for a row
 *                         whose keys are all masked (its o and residual are 0)
 */
tri_attn_status tri_attn_fwd(const tri_attn_problem *problem,
                             const void *q, const void *k, const void *v,
                             const void *bias, const uint8_t *mask,
                             void *o, void *o_residual, float *lse,
                             hipStream_t stream);

/* Device workspace (bytes) tri_attn_bwd needs for `problem`; 0 if the problem
 * is invalid or unsupported. */
size_t tri_attn_bwd_workspace_bytes(const tri_attn_problem *problem);

/*
 * Backward pass (Lambda post, "Как работает TurboPairFormer", first and third
 * points; biocloudservice page, "它优化了什么"): every probability tile is
 * recomputed once from lse and used for all four gradients; the softmax
 * correction D = rowsum(dO * O) is formed in fp32 from o plus o_residual; the
 * key, value, query and pair-bias gradients are reduced in a fixed order and
 * the full score gradient is never stored.
 *   q, k, v, bias, mask, o, lse : the forward's inputs and outputs
 *   o_residual : the forward's residual (fp32, or bf16 with the same
 *                TRI_ATTN_FLAG_RESIDUAL_BF16 as the forward); NULL = uncompensated
 *                correction D = rowsum(dO * float(o))
 *   d_o        : bf16 upstream gradient of o
 *   dq, dk, dv : bf16 gradients, [B,N,N,H,D]
 *   dbias      : [B,H,N,N] gradient of the pair bias (bf16, or fp32 with
 *                TRI_ATTN_FLAG_DBIAS_FP32)
 *   workspace  : device scratch of at least tri_attn_bwd_workspace_bytes(problem)
 *                bytes, 256-byte aligned; its contents on entry do not matter
 */
tri_attn_status tri_attn_bwd(const tri_attn_problem *problem,
                             const void *q, const void *k, const void *v,
                             const void *bias, const uint8_t *mask,
                             const void *o, const void *o_residual, const float *lse,
                             const void *d_o,
                             void *dq, void *dk, void *dv, void *dbias,
                             void *workspace, size_t workspace_bytes,
                             hipStream_t stream);

/*
 * Same as tri_attn_bwd.  In addition, when main_start and main_stop are not
 * NULL, they are recorded on `stream` immediately before and after the launch
 * of the backward's main kernel (the key-block-parallel recomputation that
 * dominates the run time), so a caller can time that kernel alone with
 * hipEventElapsedTime.  The events are owned by the caller.
 */
tri_attn_status tri_attn_bwd_profiled(const tri_attn_problem *problem,
                                      const void *q, const void *k, const void *v,
                                      const void *bias, const uint8_t *mask,
                                      const void *o, const void *o_residual,
                                      const float *lse, const void *d_o,
                                      void *dq, void *dk, void *dv, void *dbias,
                                      void *workspace, size_t workspace_bytes,
                                      hipEvent_t main_start, hipEvent_t main_stop,
                                      hipStream_t stream);

/*
 * Same as tri_attn_bwd, with every kernel of the backward bracketed by events
 * so a caller can time each one with hipEventElapsedTime.  events points to
 * five caller-owned hipEvent_t (an entry may be NULL: not recorded), recorded on
 * `stream` before the statistics kernel (0), after it (1), after the main
 * kernel (2), after the dQ reduction (3) and after the dbias reduction (4).
 * events == NULL returns TRI_ATTN_ERROR_INVALID_VALUE.  The dbias reduction
 * (events 3 to 4) is the backward's bias-gradient traffic: C fp32 partials of
 * B*H*N*N values read, the bf16 (or fp32) dbias written.
 */
tri_attn_status tri_attn_bwd_timed(const tri_attn_problem *problem,
                                   const void *q, const void *k, const void *v,
                                   const void *bias, const uint8_t *mask,
                                   const void *o, const void *o_residual,
                                   const float *lse, const void *d_o,
                                   void *dq, void *dk, void *dv, void *dbias,
                                   void *workspace, size_t workspace_bytes,
                                   const hipEvent_t *events, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* TRI_ATTN_H */
