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
 *   bias, dbias                 : bf16 [B, H, N, N] (dbias fp32 with FLAG_DBIAS_FP32).
 *                                 The kernels hold the bias as fp16: a bf16 value
 *                                 with 2^-14 <= |bias| <= 65504 converts exactly,
 *                                 smaller magnitudes round to a multiple of 2^-24,
 *                                 finite values beyond +-65504 saturate to +-65504
 *                                 and +-inf stay infinite.  Saturation keeps the
 *                                 exact softmax when such values mask keys (a key at
 *                                 -65504 gets zero weight next to any in-range
 *                                 logit) or shift every key of a query alike (a
 *                                 -1e9 masking bias on a whole query row); it
 *                                 differs only where one query's keys carry several
 *                                 different out-of-range values
 *   mask                        : uint8 [B, N, N], nonzero = key attended; NULL = all
 *   lse                         : fp32 [B, N, H, N], indexed [b, r, h, q] by
 *                                 attention row r and query q (natural log)
 *
 * Conventions shared by every entry point:
 *   - All tensor pointers are device pointers owned by the caller.  The library
 *     allocates nothing, frees nothing and keeps no pointer after returning.
 *   - Work is enqueued on `stream`; the call returns without synchronising.
 *   - Arguments are validated on the host before anything is enqueued (the only
 *     HIP calls before that query the current device).  On an error nothing is
 *     enqueued and no output is touched.  Unsupported sizes return
 *     TRI_ATTN_ERROR_NOT_SUPPORTED; there is no silent fallback path.
 *   - Tensor base pointers must be 16-byte aligned and outputs must not overlap
 *     inputs.
 *   - Results are bitwise deterministic for a fixed problem, build and device:
 *     every reduction runs in a fixed order and no floating-point atomics are
 *     used (Lambda post, "Как работает TurboPairFormer", third point).
 *   - The only global state is a per-device cache, held in atomics, of the
 *     device's compute-unit count (which sizes the launch plans and the backward
 *     workspace; 256, the MI355X's count, when no device can be queried) and of
 *     kernel attributes set once: calls from several threads are safe.
 */
#ifndef TRI_ATTN_H
#define TRI_ATTN_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TRI_ATTN_ABI_VERSION 4

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
    /* Attention rows of this call: [row_begin, row_end), 0 <= row_begin < row_end <= N,
     * or 0, 0 for all N rows (anything else: TRI_ATTN_ERROR_INVALID_VALUE).  Rows are
     * those of the attended frame (the second pair index for the ending node).  A call
     * on a range computes o, o_residual, lse (forward) and dq, dk, dv (backward) of
     * those rows only and leaves the other rows of these buffers untouched; dbias is
     * then the range's unreduced partial sum over its rows, sum_{i in range} dS_i, to
     * be added to the other ranges' partials by the caller (with
     * TRI_ATTN_FLAG_DBIAS_FP32, so that the partials are not rounded to bf16).  This is
     * one GPU's share of a row-sharded triangle attention; the sum over ranges of the
     * partials is the dbias of the whole problem (same fixed-order guarantee per
     * range, the cross-range order being the caller's). */
    int64_t row_begin, row_end;
} tri_attn_problem;

/* Supported sizes of this build: D == 16, 32 or 64, N a multiple of 32 with
 * 32 <= N <= 768, B >= 1, 1 <= H <= 64.  D == 16 runs the D == 32 kernels with the
 * tiles' channels 16..31 held at zero; D == 64 runs kernels with 64-channel tiles,
 * 32-query forward blocks and 32-key backward blocks (its backward workspace holds
 * N / 32 dQ partials instead of N / 64). */

/*
 * Returns TRI_ATTN_ABI_VERSION of the loaded library (biocloudservice page,
 * "当前可用环境非常窄，先做兼容性预检": the loader checks the binary it found
 * against what it was built for and stops with an error instead of compiling or
 * falling back at run time).  The Python binding refuses a library whose version
 * differs from its own, and every call refuses a problem whose abi_version field
 * differs (TRI_ATTN_ERROR_ABI_MISMATCH).  Never fails.
 */
int tri_attn_abi_version(void);

/*
 * Static, human-readable name of a status code; "unknown status" for a code this
 * library does not return; never NULL and never to be freed (biocloudservice
 * page, "一个可执行的验收清单", first point: a caller must be able to tell the fast
 * path ran, so an unsupported request is reported by name, never served by a
 * fallback).
 */
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

/*
 * Device workspace (bytes) tri_attn_bwd needs for `problem` on the current device;
 * 0 if the problem is invalid or unsupported (biocloudservice page, "它优化了什么，
 * 而不是只“少存一点张量”": the backward never writes the full score gradient
 * out).  The workspace holds the per-query statistics (-lse/alpha and -D, fp32,
 * 2*B*N*H*N values), one bf16 dQ partial per key block of 64 keys (32 keys at
 * D == 64: ceil(N/64)*B*N*N*H*D or N/32*B*N*N*H*D values) and one fp32
 * pair-bias-gradient partial per row chunk (C*B*H*N*N values,
 * C = the number of row chunks the launch plan uses on this device), each
 * 256-byte aligned.  At N = 768, H = 4, D = 32 that is 1.87 GB against the 3.6 GB
 * of one bf16 score gradient (N^3*H values).  Host-only; no HIP call except the
 * cached compute-unit query.
 */
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
 * Same as tri_attn_bwd (same validation, kernels and bits), with every kernel of
 * the backward bracketed by events so a caller can time each one with
 * hipEventElapsedTime (Lambda post, "Результаты тестирования", and the
 * biocloudservice page, "crop size不是一个普通参数": time is reported per crop
 * size, and here also per kernel).  events points to
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

/* Size of the library's fixed device buffer used by tri_attn_bwd_noalloc: 128 MiB. */
#define TRI_ATTN_NOALLOC_SCRATCH_BYTES (128u * 1024u * 1024u)

/*
 * Allocation-free backward, for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same arguments, kernels and bits as tri_attn_bwd without the workspace: the
 * workspace lives in a fixed device buffer of TRI_ATTN_NOALLOC_SCRATCH_BYTES that the
 * library holds on every device it runs on, from module load until the process
 * ends.  The call allocates and frees nothing; the caller still provides every
 * input and output.
 *   - Problems whose workspace (tri_attn_bwd_workspace_bytes) exceeds the buffer
 *     return TRI_ATTN_ERROR_INSUFFICIENT_WORKSPACE (with this build, B = 1, H = 4 and
 *     D = 32 on a 256-CU device: N <= 288).
 *   - The buffer keeps the last call's contents; every byte the kernels read is
 *     written earlier in the same call, so nothing needs clearing between calls.
 *   - All calls on one device share that device's buffer: calls that overlap in
 *     time on one device (other streams, other threads) race and must be
 *     serialised by the caller.
 *   - The first call on a device looks up the buffer's device address
 *     (hipGetSymbolAddress) and caches it; TRI_ATTN_ERROR_LAUNCH_FAILED if that fails.
 */
tri_attn_status tri_attn_bwd_noalloc(const tri_attn_problem *problem,
                                     const void *q, const void *k, const void *v,
                                     const void *bias, const uint8_t *mask,
                                     const void *o, const void *o_residual, const float *lse,
                                     const void *d_o,
                                     void *dq, void *dk, void *dv, void *dbias,
                                     hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* TRI_ATTN_H */
