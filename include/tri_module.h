/*
 * tri_module.h — C ABI of the triangle-attention module around the core (MI355X,
 * gfx950), built into the same library as tri_attn.h.
 *
 * Operation.  The pages present the kernel as triangle attention in the style of
 * AlphaFold3 (biocloudservice page, "16张H100，训练步提速1.73倍", opening paragraph)
 * and describe nothing around its attention core; the block built here is the AlphaFold3
 * triangle-attention block around the starting node, on a pair tensor z [B, N, N, C]
 * with C = H * D = 128 channels:
 *     zn      = LayerNorm(z)                  over the C channels, learned scale w and
 *                                             offset b (fp32), eps (0 = 1e-5)
 *     q, k, v = zn Wq, zn Wk, zn Wv           [B, N, N, H, D], no bias terms
 *     bias    = zn Wb                         bias[b, h, j, k] = (zn Wb)[b, j, k, h]
 *     g       = sigmoid(zn Wg)                [B, N, N, C]
 *     o       = tri_attn_fwd(q, k, v, bias, mask)
 *     y       = (g * o) Wo                    [B, N, N, C]
 * With TRI_ATTN_FLAG_ENDING_NODE it is the same block on the pair tensor with its two
 * pair axes swapped (z and the mask transposed, y transposed back): every step but the
 * core acts per position, so the bias is stored transposed,
 * bias[b, h, j, k] = (zn Wb)[b, k, j, h], and the core runs in its ending-node mode.
 * The backward returns dz and the gradients of w, b, Wq|Wk|Wv|Wg, Wb and Wo.
 *
 * Layouts (row-major, last index fastest):
 *   z, y, dy, dz, zn, g : bf16 [B, N, N, C] (one position = 256 contiguous bytes)
 *   q, k, v, o          : bf16 [B, N, N, H, D], the core's layout (the same bytes as
 *                         [B, N, N, C] with channel h * D + d)
 *   bias                : bf16 [B, H, N, N], the pair bias as the core takes it
 *   o_residual          : fp32 [B, N, N, H, D];  lse : fp32 [B, N, H, N] (see tri_attn.h)
 *   ln_stats            : fp32 [B, N, N, 2]: mean and 1 / sqrt(variance + eps) per position
 *   ln_w, ln_b          : fp32 [C]
 *   w_qkvg              : bf16 [C, 4 C]: Wq | Wk | Wv | Wg side by side, column
 *                         128 * block + h * D + d
 *   w_bias              : bf16 [C, H];  w_out : bf16 [C, C] (row = channel h * D + d of o)
 *   gradients           : fp32, the shapes of their parameters; dz bf16
 *   mask                : uint8 [B, N, N] as in tri_attn.h, or NULL
 *
 * Precision: every matrix product takes bf16 operands (zn, the gated output, the
 * gradients) and accumulates in fp32; LayerNorm statistics, the gate and the LayerNorm
 * backward are fp32; position outputs are round-to-nearest-even bf16.  Every sum runs
 * in a fixed order, so results are bitwise reproducible (Lambda post, "Как работает
 * TurboPairFormer", third point); the weight gradients are sums over all B N N
 * positions, taken as fixed slices whose fp32 partials are added in slice order.
 *
 * Conventions as in tri_attn.h: caller-owned device pointers, 16-byte aligned; every
 * output (the saved activations of the forward, the gradients and the workspace of the
 * backward) must not overlap any input or other output (checked: TRI_ATTN_ERROR_INVALID_
 * VALUE before anything is enqueued); work enqueued on
 * `stream`, no synchronisation; host-side validation before anything is enqueued.
 * Supported: H * D == 128 with the core's supported H and D, the core's N (a multiple
 * of 32 up to 768), any B; other sizes return TRI_ATTN_ERROR_NOT_SUPPORTED.
 */
#ifndef TRI_MODULE_H
#define TRI_MODULE_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#include "tri_attn.h"

#ifdef __cplusplus
extern "C" {
#endif

#define TRI_ATTN_MODULE_ABI_VERSION 1

typedef struct {
    int32_t abi_version;  /* must equal TRI_ATTN_MODULE_ABI_VERSION */
    int32_t flags;        /* 0 or TRI_ATTN_FLAG_ENDING_NODE */
    int64_t B, N, H, D;   /* batch, pair length, heads, head dim (H * D == 128) */
    float ln_eps;         /* LayerNorm epsilon; 0 => 1e-5 */
} tri_attn_module_problem;

/* Parameters (device pointers). */
typedef struct {
    const float *ln_w, *ln_b;   /* fp32 [C] */
    const void *w_qkvg;         /* bf16 [C, 4 C] */
    const void *w_bias;         /* bf16 [C, H] */
    const void *w_out;          /* bf16 [C, C] */
} tri_attn_module_params;

/* The forward's saved activations (device pointers): written by tri_attn_module_fwd,
 * read by tri_attn_module_bwd. */
typedef struct {
    void *zn;          /* bf16 [B, N, N, C] */
    float *ln_stats;   /* fp32 [B, N, N, 2] */
    void *q, *k, *v;   /* bf16 [B, N, N, H, D] */
    void *g;           /* bf16 [B, N, N, C] */
    void *bias;        /* bf16 [B, H, N, N] */
    void *o;           /* bf16 [B, N, N, H, D] */
    float *o_residual; /* fp32 [B, N, N, H, D] */
    float *lse;        /* fp32 [B, N, H, N] */
} tri_attn_module_saved;

/* Parameter gradients (device pointers, fp32, overwritten). */
typedef struct {
    float *ln_w, *ln_b;  /* [C] */
    float *w_qkvg;       /* [C, 4 C] */
    float *w_bias;       /* [C, H] */
    float *w_out;        /* [C, C] */
} tri_attn_module_param_grads;

/* Returns TRI_ATTN_MODULE_ABI_VERSION of the loaded library (biocloudservice page,
 * "当前可用环境非常窄，先做兼容性预检": the interface is checked, not assumed). */
int tri_attn_module_abi_version(void);

/*
 * Forward of the block (biocloudservice page, "16张H100，训练步提速1.73倍", opening
 * paragraph: triangle attention in the style of AlphaFold3; the core as in
 * tri_attn_fwd): y from z, the mask and the
 * parameters; fills every field of `saved`.  Returns the core's status where it
 * rejects the problem.
 */
tri_attn_status tri_attn_module_fwd(const tri_attn_module_problem *problem, const void *z,
                                    const uint8_t *mask, const tri_attn_module_params *params,
                                    void *y, const tri_attn_module_saved *saved,
                                    hipStream_t stream);

/*
 * Device workspace (bytes) tri_attn_module_bwd needs: dO and the gate gradient, the
 * core's dq, dk, dv (bf16 position tensors) and fp32 dbias, the core's own workspace
 * (tri_attn_bwd_workspace_bytes, biocloudservice page, "它优化了什么": no full score
 * gradient), the weight gradients' slice partials and the LayerNorm gradients' tile
 * partials, each 256-byte aligned; 0 for an invalid or unsupported problem.
 */
size_t tri_attn_module_bwd_workspace_bytes(const tri_attn_module_problem *problem);

/*
 * Backward of the block (Lambda post, "Как работает TurboPairFormer", first and third
 * points: the core's four gradients from one probability recompute, fixed-order
 * accumulation everywhere): dz and the parameter gradients from dy and the forward's
 * saved activations.  `workspace` must be 256-byte aligned and at least
 * tri_attn_module_bwd_workspace_bytes; TRI_ATTN_ERROR_INSUFFICIENT_WORKSPACE otherwise.
 */
tri_attn_status tri_attn_module_bwd(const tri_attn_module_problem *problem, const void *z,
                                    const uint8_t *mask, const tri_attn_module_params *params,
                                    const tri_attn_module_saved *saved, const void *dy, void *dz,
                                    const tri_attn_module_param_grads *grads, void *workspace,
                                    size_t workspace_bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* TRI_MODULE_H */
