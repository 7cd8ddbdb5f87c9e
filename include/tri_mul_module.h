/*
 * tri_mul_module.h — C ABI of the triangle multiplicative update block around its
 * contraction (MI355X, gfx950), built into the same library as tri_mul.h.
 *
 * Operation.  The pages name the triangle multiplicative update as the method's second
 * kernel family (biocloudservice page, "16张H100，训练步提速1.73倍", opening paragraph;
 * Lambda post, "TurboPairFormer: более быстрое, стабильное и точное дообучение
 * OpenFold3", opening section) and describe nothing of it; the block built here is
 * the AlphaFold3 triangle multiplicative update, on a pair tensor z [B, N, N, C] with
 * C = 128 channels and a pair mask m [B, N, N]:
 *     zn = LayerNorm_in(z)                 learned scale and offset (fp32), eps (0 = 1e-5)
 *     a  = sigmoid(zn Wag) * (zn Wap) * m  no bias terms; hidden width C
 *     b  = sigmoid(zn Wbg) * (zn Wbp) * m
 *     g  = sigmoid(zn Wg)
 *     x  = tri_mul_fwd(a, b)               outgoing, or incoming with TRI_MUL_FLAG_INCOMING
 *     y  = g * (LayerNorm_out(x) Wo)
 * The backward returns dz and the gradients of both LayerNorms' scale and offset, of
 * Wag | Wap | Wbg | Wbp | Wg and of Wo.
 *
 * Layouts (row-major, last index fastest):
 *   z, y, dy, dz, zn, g, xn : bf16 [B, N, N, C] (one position = 256 contiguous bytes)
 *   a, b, x                 : bf16 [B, C, N, N], channel-major as in tri_mul.h
 *   ln_in_stats, ln_out_stats : fp32 [B, N, N, 2]: mean and 1 / sqrt(variance + eps)
 *   ln_*_w, ln_*_b          : fp32 [C]
 *   w_in                    : bf16 [C, 5 C]: Wag | Wap | Wbg | Wbp | Wg side by side
 *   w_out                   : bf16 [C, C]
 *   gradients               : fp32, the shapes of their parameters; dz bf16
 *   mask                    : uint8 [B, N, N] (nonzero = kept), or NULL for all kept
 *
 * Precision: matrix products take bf16 operands and accumulate in fp32; LayerNorm
 * statistics, gates and LayerNorm backwards are fp32; position outputs, a, b and the
 * contraction are round-to-nearest-even bf16.  Every sum runs in a fixed order
 * (bitwise reproducible; Lambda post, "Как работает TurboPairFormer", third point).
 *
 * Conventions as in tri_attn.h: caller-owned device pointers, 16-byte aligned; every
 * output (the saved activations of the forward, the gradients and the workspace of the
 * backward) must not overlap any input or other output (checked: TRI_ATTN_ERROR_INVALID_
 * VALUE before anything is enqueued); work enqueued on `stream`;
 * host-side validation before anything is enqueued.  Supported: C == 128, N a multiple
 * of 32 up to 1024, B * C <= 65536; otherwise TRI_ATTN_ERROR_NOT_SUPPORTED.
 */
#ifndef TRI_MUL_MODULE_H
#define TRI_MUL_MODULE_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#include "tri_attn.h"
#include "tri_mul.h"

#ifdef __cplusplus
extern "C" {
#endif

#define TRI_MUL_MODULE_ABI_VERSION 1

typedef struct {
    int32_t abi_version;  /* must equal TRI_MUL_MODULE_ABI_VERSION */
    int32_t flags;        /* 0 or TRI_MUL_FLAG_INCOMING */
    int64_t B, N, C;      /* batch, pair length, channels (C == 128) */
    float ln_eps;         /* both LayerNorms' epsilon; 0 => 1e-5 */
} tri_mul_module_problem;

typedef struct {
    const float *ln_in_w, *ln_in_b;   /* fp32 [C] */
    const void *w_in;                 /* bf16 [C, 5 C] */
    const float *ln_out_w, *ln_out_b; /* fp32 [C] */
    const void *w_out;                /* bf16 [C, C] */
} tri_mul_module_params;

/* The forward's saved activations: written by tri_mul_module_fwd, read by the backward. */
typedef struct {
    void *zn;            /* bf16 [B, N, N, C] */
    float *ln_in_stats;  /* fp32 [B, N, N, 2] */
    void *a, *b;         /* bf16 [B, C, N, N] */
    void *g;             /* bf16 [B, N, N, C] */
    void *x;             /* bf16 [B, C, N, N] */
    void *xn;            /* bf16 [B, N, N, C] */
    float *ln_out_stats; /* fp32 [B, N, N, 2] */
} tri_mul_module_saved;

typedef struct {
    float *ln_in_w, *ln_in_b;   /* [C] */
    float *w_in;                /* [C, 5 C] */
    float *ln_out_w, *ln_out_b; /* [C] */
    float *w_out;               /* [C, C] */
} tri_mul_module_param_grads;

/* Returns TRI_MUL_MODULE_ABI_VERSION of the loaded library (biocloudservice page,
 * "当前可用环境非常窄，先做兼容性预检": the interface is checked, not assumed). */
int tri_mul_module_abi_version(void);

/*
 * Forward of the block (biocloudservice page, "16张H100，训练步提速1.73倍", opening
 * paragraph: the triangle multiplicative update as the second kernel family): y from
 * z, the mask and the parameters; fills every field of `saved`.
 */
tri_attn_status tri_mul_module_fwd(const tri_mul_module_problem *problem, const void *z,
                                   const uint8_t *mask, const tri_mul_module_params *params,
                                   void *y, const tri_mul_module_saved *saved,
                                   hipStream_t stream);

/*
 * Device workspace (bytes) tri_mul_module_bwd needs (biocloudservice page, "它优化了什么":
 * intermediate gradients kept to what the fixed-order reductions need): the output
 * projection's and gate's gradients, dx, da, db and the four projection gradients (bf16,
 * one position tensor each), the weight gradients' slice partials and both LayerNorms'
 * tile partials, each 256-byte aligned; 0 for an invalid or unsupported problem.
 */
size_t tri_mul_module_bwd_workspace_bytes(const tri_mul_module_problem *problem);

/*
 * Backward of the block (Lambda post, "Как работает TurboPairFormer", third point:
 * fixed-order accumulation, no floating-point atomics): dz and the parameter gradients
 * from dy and the saved activations.  `workspace` must be 256-byte aligned and at
 * least tri_mul_module_bwd_workspace_bytes.
 */
tri_attn_status tri_mul_module_bwd(const tri_mul_module_problem *problem, const void *z,
                                   const uint8_t *mask, const tri_mul_module_params *params,
                                   const tri_mul_module_saved *saved, const void *dy, void *dz,
                                   const tri_mul_module_param_grads *grads, void *workspace,
                                   size_t workspace_bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* TRI_MUL_MODULE_H */
