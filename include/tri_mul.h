/*
 * tri_mul.h — C ABI of the triangle multiplicative update's contraction (MI355X,
 * gfx950), built into the same library as tri_attn.h.
 *
 * Operation (TurboPairFormer pages: the biocloudservice page's opening paragraph and
 * the Lambda post's opening section name the triangle multiplicative update as the
 * method's second kernel family; they do not write it out).  Its cubic-cost core, per
 * batch b and channel c, contracts two projected pair tensors a and bb over the third
 * node of every triangle:
 *     outgoing edges: z[i, j] = sum_k a[i, k] * bb[j, k]
 *     incoming edges: z[i, j] = sum_k a[k, i] * bb[k, j]       (TRI_MUL_FLAG_INCOMING)
 * and the backward returns, for g = dL/dz,
 *     outgoing: da[i, k] = sum_j g[i, j] bb[j, k],   dbb[j, k] = sum_i g[i, j] a[i, k]
 *     incoming: da[k, i] = sum_j g[i, j] bb[k, j],   dbb[k, j] = sum_i g[i, j] a[k, i]
 * (The block's projections, sigmoid gates, masks and layer norms, which act per
 * position before and after the contraction, are not part of this library.)
 *
 * Layout: every tensor is bf16, channel-major [B, C, N, N] (row-major, last index
 * fastest): one N x N matrix per (batch, channel), in which each product above is a
 * dense matrix product.  Accumulation is fp32 in one fixed order per output value
 * (bitwise reproducible, no atomics); outputs are round-to-nearest-even bf16.
 *
 * Conventions as in tri_attn.h: caller-owned device pointers, 16-byte aligned, outputs
 * not overlapping inputs; work enqueued on `stream`, no synchronisation; host-side
 * validation before anything is enqueued; unsupported sizes return
 * TRI_ATTN_ERROR_NOT_SUPPORTED.  Supported: N a multiple of 32, N <= 1024,
 * B * C <= 65536.
 */
#ifndef TRI_MUL_H
#define TRI_MUL_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#include "tri_attn.h"

#ifdef __cplusplus
extern "C" {
#endif

#define TRI_MUL_ABI_VERSION 1

enum {
    TRI_MUL_FLAG_INCOMING = 1 << 0  /* incoming edges (default: outgoing edges) */
};

typedef struct {
    int32_t abi_version;  /* must equal TRI_MUL_ABI_VERSION */
    int32_t flags;        /* TRI_MUL_FLAG_* */
    int64_t B, N, C;      /* batch, pair length, channels */
} tri_mul_problem;

/* Returns TRI_MUL_ABI_VERSION of the loaded library (biocloudservice page,
 * "当前可用环境非常窄，先做兼容性预检": the binary's interface is checked, not assumed). */
int tri_mul_abi_version(void);

/*
 * Forward contraction (biocloudservice page, "16张H100，训练步提速1.73倍", opening
 * paragraph: the triangle multiplicative update named next to triangle attention):
 * z from a and bb, all bf16 [B, C, N, N].
 */
tri_attn_status tri_mul_fwd(const tri_mul_problem *problem, const void *a, const void *bb, void *z,
                            hipStream_t stream);

/*
 * Backward contraction (Lambda post, "TurboPairFormer: более быстрое, стабильное и
 * точное дообучение OpenFold3", opening section: the method's triangle multiplication
 * next to its attention; "Как работает TurboPairFormer", third point: fixed-order
 * accumulation): da and dbb from a, bb and dz = dL/dz, all bf16 [B, C, N, N]; two
 * matrix products per (batch, channel), each one fixed-order sum per output value.
 */
tri_attn_status tri_mul_bwd(const tri_mul_problem *problem, const void *a, const void *bb, const void *dz,
                            void *da, void *dbb, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* TRI_MUL_H */
