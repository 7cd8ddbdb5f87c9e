// The triangle-attention module around the core, forward and backward, for MI355X
// (gfx950, CDNA4).
//
// Operation (reading of the biocloudservice page's opening paragraph, which presents the
// kernel as triangle attention in the style of AlphaFold3 and describes nothing around
// the core): on a pair tensor
// z [B, N, N, C], C = H * D = 128,
//   zn = LayerNorm(z);  q, k, v = zn Wq, zn Wk, zn Wv;  bias[b,h,j,k] = (zn Wb)[b,j,k,h]
//   g = sigmoid(zn Wg);  o = core(q, k, v, bias, mask);  y = (g * o) Wo
// (no bias terms in the projections); the ending-node block is the same block on the
// transposed pair tensor, i.e. the bias transposed (bias[b,h,j,k] = (zn Wb)[b,k,j,h])
// and the core run with its ending-node flag.
//
// Every step but the core is per position, so the kernels work on tiles of 128
// consecutive positions (rows of the [B N N, 128] matrices) times 128 x 128 weight
// blocks, one v_mfma_f32_32x32x16_bf16 tile product per workgroup (4 waves, 2 x 2 of
// 64 x 64), with the prologue or epilogue fused:
//   mod_proj        LayerNorm in (statistics per position in fp32), zn into LDS; then
//                   the q, k, v, gate (sigmoid) and bias (transposed store) blocks out
//   mod_gate_out    bf16(g * o) in, y out
//   mod_out_bwd     dy Wo^T; out: dO = dgo * g and the gate's pre-activation gradient
//                   dgo * o * g (1 - g)
//   mod_in_bwd      dzn = [dq dk dv dg] Wqkvg^T + dbias Wb^T (five 128-deep steps);
//                   the LayerNorm backward out, and per-tile partial sums of the
//                   LayerNorm scale and offset gradients
//   mod_wgrad       weight gradients zn^T [dq dk dv dg dbias] and bf16(g * o)^T dy:
//                   contractions over all positions, split into fixed slices whose fp32
//                   partials the reduction kernels sum in slice order
// No floating-point atomics: every result is one fixed-order sum (bitwise reproducible,
// as the core: Lambda post, "Как работает TurboPairFormer", third point).
//
// MFMA layouts (64 lanes, hh = lane / 32):
//   A (32 x 16): lane supplies A[lane % 32][8 hh + e], e = 0..7
//   B (16 x 32): lane supplies B[8 hh + e][lane % 32]
//   C (32 x 32): lane holds C[8 (r / 4) + 4 hh + r % 4][lane % 32], r = 0..15
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <type_traits>
#include <math.h>
#include <string.h>

#include "tri_attn.h"
#include "tri_module.h"
#include "tri_mul.h"
#include "tri_mul_module.h"

namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) unsigned u32x4;
typedef __attribute__((ext_vector_type(4))) short i16x4;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr int CH = 128;   // pair channels (H * D)
constexpr int TP = 128;   // positions per tile
constexpr int NT = 256;   // threads per workgroup (4 waves)
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ unsigned pack_bf16(float a, float b) {
  return __builtin_bit_cast(unsigned, __builtin_convertvector((f32x2){a, b}, bf16x2));
}
__device__ __forceinline__ float bf_lo(unsigned w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(unsigned w) { return __uint_as_float(w & 0xffff0000u); }

// Element (row, col) of a [128][128] bf16 LDS tile.  The 16-byte chunks of a row are
// permuted by ((row & 3) << 2) | ((row >> 2) & 3): the 16-byte row reads of 16
// consecutive rows (one chunk each) touch all 64 banks once, and so do the transposing
// reads, whose 16-lane groups cover rows 4t .. 4t + 3 over two consecutive chunks (the
// four rows map the chunk pair to four disjoint bank groups).
__device__ __forceinline__ int toff(int row, int col) {
  const int sw = ((row & 3) << 2) | ((row >> 2) & 3);
  return row * 128 + (((col >> 3) ^ sw) << 3) + (col & 7);
}
// Row operand: lane gets tile[row0 + lane % 32][kk + 8 hh + e].
__device__ __forceinline__ bf16x8 row_operand(const uint16_t *tile, int row0, int kk, int lane) {
  return *(const bf16x8 *)(tile + toff(row0 + (lane & 31), kk + 8 * (lane >> 5)));
}
// Transposed operand: lane gets tile[kk + 8 hh + e][col0 + lane % 32].  ds_read_b64_tr_b16
// works on 4 x 16 blocks: in each 16-lane group, lane 4 m + s addresses row m, columns
// 4 s .. 4 s + 3, and lane c of the group receives column c of the four rows.
__device__ __forceinline__ bf16x8 tr_operand(const uint16_t *tile, int kk, int col0, int lane) {
  const int g = lane >> 4, w = lane & 15, m = w >> 2, s = w & 3;
  const int row = kk + 8 * (lane >> 5) + m, col = col0 + 16 * (g & 1) + 4 * s;
  i16x4 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(tile + toff(row, col)));
  i16x4 y = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(tile + toff(row + 4, col)));
  typedef __attribute__((ext_vector_type(8))) short i16x8;
  return __builtin_bit_cast(bf16x8, (i16x8)__builtin_shufflevector(x, y, 0, 1, 2, 3, 4, 5, 6, 7));
}

// How an operand sits in its LDS tile: ROW = [m or n][t] (contraction index
// contiguous), TR = [t][m or n].
enum Layout { ROW = 0, TR = 1 };

// acc[i][j] += sum over t in [0, 16 * slices) of A(wm + 32 i + ., t) B(t, wn + 32 j + .).
// MI = 2: a wave owns 64 x 64 of the 128 x 128 tile (4 waves); MI = 1: 32 x 64 (8 waves).
template <int AL, int BL, int MI = 2>
__device__ __forceinline__ void tile_product(const uint16_t *sA, const uint16_t *sB, int wm, int wn, int lane,
                                             int slices, f32x16 (&acc)[MI][2]) {
  for (int s = 0; s < slices; ++s) {
    const int kk = 16 * s;
    bf16x8 a[MI], b[2];
#pragma unroll
    for (int i = 0; i < MI; ++i)
      a[i] = AL == ROW ? row_operand(sA, wm + 32 * i, kk, lane) : tr_operand(sA, kk, wm + 32 * i, lane);
#pragma unroll
    for (int j = 0; j < 2; ++j)
      b[j] = BL == ROW ? row_operand(sB, wn + 32 * j, kk, lane) : tr_operand(sB, kk, wn + 32 * j, lane);
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) acc[i][j] = mfma(a[i], b[j], acc[i][j]);
  }
}

// tile_product for one 32 x 64 block per wave with its 16-deep slices unrolled two at
// a time, which bounds how far ahead their LDS reads are hoisted (fewer registers)
template <int AL, int BL>
__device__ __forceinline__ void tile_product_u2(const uint16_t *sA, const uint16_t *sB, int wm, int wn, int lane,
                                                int slices, f32x16 (&acc)[1][2]) {
#pragma unroll 2
  for (int s = 0; s < slices; ++s) {
    const int kk = 16 * s;
    const bf16x8 a = AL == ROW ? row_operand(sA, wm, kk, lane) : tr_operand(sA, kk, wm, lane);
    bf16x8 b[2];
#pragma unroll
    for (int j = 0; j < 2; ++j)
      b[j] = BL == ROW ? row_operand(sB, wn + 32 * j, kk, lane) : tr_operand(sB, kk, wn + 32 * j, lane);
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[0][j] = mfma(a, b[j], acc[0][j]);
  }
}

template <int MI = 2>
__device__ __forceinline__ void zero(f32x16 (&acc)[MI][2]) {
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = (f32x16){};
}

// A [128][128] bf16 matrix block (rows row0.., 256-byte rows of a row-major matrix with
// `ld` elements per row, columns col0 .. col0 + 127) into an LDS tile: thread t of T
// copies 16-byte pieces t, t + T, ...
template <int T = NT>
__device__ __forceinline__ void load_block(uint16_t *tile, const uint16_t *src, long long ld, int tid) {
#pragma unroll
  for (int i = 0; i < 2048 / T; ++i) {
    const int p = tid + T * i, row = p >> 4, c = (p & 15) * 8;
    *(u32x4 *)(tile + toff(row, c)) = *(const u32x4 *)(src + (long long)row * ld + c);
  }
}

// load_block in two halves, so that the loads can be in flight while the workgroup
// computes: fetch_block issues them into registers, put_block writes those to the tile.
template <int T>
__device__ __forceinline__ void fetch_block(u32x4 (&r)[2048 / T], const uint16_t *src, long long ld, int tid) {
#pragma unroll
  for (int i = 0; i < 2048 / T; ++i) {
    const int p = tid + T * i, row = p >> 4, c = (p & 15) * 8;
    r[i] = *(const u32x4 *)(src + (long long)row * ld + c);
  }
}
template <int T>
__device__ __forceinline__ void put_block(uint16_t *tile, const u32x4 (&r)[2048 / T], int tid) {
#pragma unroll
  for (int i = 0; i < 2048 / T; ++i) {
    const int p = tid + T * i, row = p >> 4, c = (p & 15) * 8;
    *(u32x4 *)(tile + toff(row, c)) = r[i];
  }
}

// The accumulator tile as bf16 into an LDS tile (f applied to each value), then stored
// as 128 rows of 256 bytes to dst (row stride 128 elements) by the workgroup's T threads.
template <int MI = 2, int T = NT, typename F>
__device__ __forceinline__ void store_tile_bf16(uint16_t *tile, uint16_t *dst, const f32x16 (&acc)[MI][2], int wm,
                                                int wn, int lane, int tid, F f) {
  const int hh = lane >> 5, ll = lane & 31;
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = wm + 32 * i + 8 * (r >> 2) + 4 * hh + (r & 3), n = wn + 32 * j + ll;
        tile[toff(m, n)] = (uint16_t)(pack_bf16(f(acc[i][j][r]), 0.f) & 0xffffu);
      }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 2048 / T; ++i) {
    const int p = tid + T * i, row = p >> 4, c = (p & 15) * 8;
    *(u32x4 *)(dst + (long long)row * CH + c) = *(const u32x4 *)(tile + toff(row, c));
  }
}

// fp32 [128][128] LDS tile for epilogues that need whole position rows: element (row,
// col) at row * 128 + (col ^ 4 * (row & 7)) (4-byte granules permuted in groups of
// four so that the accumulator writes of the two lane halves use different banks).
__device__ __forceinline__ int foff(int row, int col) { return row * 128 + (col ^ ((row & 7) << 2)); }

template <int MI = 2, typename F>
__device__ __forceinline__ void stage_f32(float *t32, const f32x16 (&acc)[MI][2], int wm, int wn, int lane, F f) {
  const int hh = lane >> 5, ll = lane & 31;
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = wm + 32 * i + 8 * (r >> 2) + 4 * hh + (r & 3), n = wn + 32 * j + ll;
        t32[foff(m, n)] = f(acc[i][j][r]);
      }
}
// 8 consecutive columns c .. c + 7 (c a multiple of 8) of row `row` of a foff tile
__device__ __forceinline__ void read8_f32(const float *t32, int row, int c, float *x) {
  const f32x4 a = *(const f32x4 *)(t32 + foff(row, c)), b = *(const f32x4 *)(t32 + foff(row, c + 4));
  x[0] = a[0]; x[1] = a[1]; x[2] = a[2]; x[3] = a[3];
  x[4] = b[0]; x[5] = b[1]; x[6] = b[2]; x[7] = b[3];
}

__device__ __forceinline__ void unpack8(u32x4 w, float *x) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = bf_lo(w[i]);
    x[2 * i + 1] = bf_hi(w[i]);
  }
}
__device__ __forceinline__ u32x4 pack8u(const float *x) {
  return (u32x4){pack_bf16(x[0], x[1]), pack_bf16(x[2], x[3]), pack_bf16(x[4], x[5]), pack_bf16(x[6], x[7])};
}

__device__ __forceinline__ float sigmoidf_(float x) { return 1.f / (1.f + __builtin_amdgcn_exp2f(-x * kLog2e)); }

// Workgroup index -> tile index such that consecutive tiles share an XCD.
__device__ __forceinline__ int xcd_remap(int L, int G) {
  const int per = G >> 3;
  if (L < (per << 3)) return (L & 7) * per + (L >> 3);
  return L;
}

constexpr int NT8 = 512;  // threads of the 8-wave kernels (two waves per SIMD)

// Column sums over the tile's 128 positions of an fp32 foff tile by 512 threads (thread
// -> channel tid % 128, quarter tid / 128 of the positions in order, then the quarters
// in order): channel c's sum to dst[c].  Ends with the workgroup synchronised.
__device__ __forceinline__ void column_sums8(const float *t32, float (*s_part)[CH], float *dst, int tid) {
  const int c = tid & 127, q = tid >> 7;
  float sum = 0.f;
#pragma unroll 16
  for (int r = 32 * q; r < 32 * q + 32; ++r) sum += t32[foff(r, c)];
  s_part[q][c] = sum;
  __syncthreads();
  if (q == 0) dst[c] = ((s_part[0][c] + s_part[1][c]) + s_part[2][c]) + s_part[3][c];
  __syncthreads();
}

struct ModArgs {
  // forward
  const uint16_t *z;
  const float *ln_w, *ln_b;
  const uint16_t *w_qkvg, *w_bias, *w_out;
  uint16_t *zn;
  float *stats;                // [P][2]: mean, rstd
  uint16_t *q, *k, *v, *g, *bias, *o, *y;
  // backward
  const uint16_t *dy;
  uint16_t *d_o, *dgp;         // dO for the core, the gate's pre-activation gradient
  const uint16_t *dq, *dk, *dv;
  const float *dbias;          // fp32 [B, H, N, N] (the core's frame)
  uint16_t *dz;
  float *ln_part;              // [tiles][2][128]: per-tile sums of dzn * xhat and dzn
  float *w_part;               // [6][S][128][128]
  int B, N, H, ending;
  long long P;                 // positions B N N
  int tiles, slices;
  float eps;
};

// The bias elements of one tile of 128 positions p0 + row: every position of a tile
// lies in one batch b (N^2 is a multiple of 1024), so the tile's pair-bias offsets are
//   bias[b, h, j, k] = base + h N^2 + (j N + k)    (starting node, position (b, j, k))
//   bias[b, h, k, j] = base + h N^2 + (k N + j)    (ending node)
// with base = b H N^2 and 32-bit position offsets within the batch.
struct BiasTile {
  long long base, nn;
  int jk0, n, ending;
  __device__ BiasTile(const ModArgs &a, long long p0) {
    nn = (long long)a.N * a.N;
    const long long b = p0 / nn;
    base = b * a.H * nn;
    jk0 = (int)(p0 - b * nn);
    n = a.N;
    ending = a.ending;
  }
  __device__ long long at(int row, int h) const {
    const int jk = jk0 + row;
    int e = jk;
    if (ending) {
      const int j = jk / n;
      e = (jk - j * n) * n + j;
    }
    return base + h * nn + e;
  }
};

// ------------------------------------------------------------------------------------
// Forward
// ------------------------------------------------------------------------------------
// Workgroup = one tile of 128 positions: the LayerNorm once (zn into LDS, and with the
// statistics to HBM for the backward), then the five output blocks in turn (q, k, v,
// the gate, the bias), each a 128 x 128 weight block times the zn tile.  The next
// block's weights are loaded into registers while the current block's products run;
// each block's output leaves through the weight tile's LDS space once the products
// are done.
__global__ __launch_bounds__(NT, 2) void mod_proj_kernel(ModArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t sA[TP * CH];
  __shared__ __attribute__((aligned(16))) uint16_t sB[CH * CH];
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const long long p0 = (long long)xcd_remap(blockIdx.x, gridDim.x) * TP;

  // weights of block blk (< 4) as 16-byte pieces: B[t = input channel][n = output column]
  u32x4 wr[8];
  auto fetch_w = [&](int blk) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int pc = tid + NT * i, row = pc >> 4, c = (pc & 15) * 8;
      wr[i] = *(const u32x4 *)(a.w_qkvg + (long long)row * 4 * CH + blk * CH + c);
    }
  };
  auto stage_w = [&]() {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int pc = tid + NT * i, row = pc >> 4, c = (pc & 15) * 8;
      *(u32x4 *)(sB + toff(row, c)) = wr[i];
    }
  };
  fetch_w(0);  // in flight during the LayerNorm
  // LayerNorm: thread -> position tid / 2, channels 64 (tid % 2) .. + 63
  {
    const int pr = tid >> 1, c0 = 64 * (tid & 1);
    const uint16_t *src = a.z + (p0 + pr) * CH + c0;
    float x[64];
#pragma unroll
    for (int i = 0; i < 8; ++i) unpack8(*(const u32x4 *)(src + 8 * i), x + 8 * i);
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 64; ++i) s += x[i];
    s += __shfl_xor(s, 1);
    const float mean = s * (1.f / CH);
    float v = 0.f;
#pragma unroll
    for (int i = 0; i < 64; ++i) {
      const float d = x[i] - mean;
      v = fmaf(d, d, v);
    }
    v += __shfl_xor(v, 1);
    const float rstd = 1.f / sqrtf(v * (1.f / CH) + a.eps);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float y8[8];
      const f32x4 w0 = *(const f32x4 *)(a.ln_w + c0 + 8 * i), w1 = *(const f32x4 *)(a.ln_w + c0 + 8 * i + 4);
      const f32x4 b0 = *(const f32x4 *)(a.ln_b + c0 + 8 * i), b1 = *(const f32x4 *)(a.ln_b + c0 + 8 * i + 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        y8[e] = fmaf((x[8 * i + e] - mean) * rstd, w0[e], b0[e]);
        y8[4 + e] = fmaf((x[8 * i + 4 + e] - mean) * rstd, w1[e], b1[e]);
      }
      const u32x4 w = pack8u(y8);
      *(u32x4 *)(sA + toff(pr, c0 + 8 * i)) = w;
      *(u32x4 *)(a.zn + (p0 + pr) * CH + c0 + 8 * i) = w;
    }
    if ((tid & 1) == 0) *(f32x2 *)(a.stats + 2 * (p0 + pr)) = (f32x2){mean, rstd};
  }
  stage_w();
  __syncthreads();

  const int wm = (wave >> 1) * 64, wn = (wave & 1) * 64;
#pragma unroll 1
  for (int blk = 0; blk < 5; ++blk) {
    if (blk + 1 < 4) fetch_w(blk + 1);  // in flight during the products
    f32x16 acc[2][2];
    zero(acc);
    tile_product<ROW, TR>(sA, sB, wm, wn, lane, CH / 16, acc);
    __syncthreads();  // every wave is done with the weight tile
    if (blk < 3) {
      uint16_t *dst = (blk == 0 ? a.q : blk == 1 ? a.k : a.v) + p0 * CH;
      store_tile_bf16(sB, dst, acc, wm, wn, lane, tid, [](float x) { return x; });
    } else if (blk == 3) {
      store_tile_bf16(sB, a.g + p0 * CH, acc, wm, wn, lane, tid, [](float x) { return sigmoidf_(x); });
    } else {
      // the bias: column n < H is head n
      const int hh = lane >> 5, ll = lane & 31;
      const BiasTile bt(a, p0);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int n = wn + 32 * j + ll;
          if (n >= a.H) continue;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int m = wm + 32 * i + 8 * (r >> 2) + 4 * hh + (r & 3);
            a.bias[bt.at(m, n)] = (uint16_t)(pack_bf16(acc[i][j][r], 0.f) & 0xffffu);
          }
        }
      break;
    }
    __syncthreads();  // the staged output is read back
    if (blk + 1 < 4) {
      stage_w();
    } else {
      // the bias block's weights: Wb[c_in][h] in the H head columns, zeros elsewhere
      const u32x4 z4 = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int pc = tid + NT * i, row = pc >> 4, c = (pc & 15) * 8;
        *(u32x4 *)(sB + toff(row, c)) = z4;
      }
      __syncthreads();
      for (int e = tid; e < CH * a.H; e += NT) {
        const int row = e / a.H, h = e - row * a.H;
        sB[toff(row, h)] = a.w_bias[e];
      }
    }
    __syncthreads();
  }
}

// y = bf16(g * o) Wo, one workgroup per tile of 128 positions.
__global__ __launch_bounds__(NT, 2) void mod_gate_out_kernel(ModArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t sA[TP * CH];
  __shared__ __attribute__((aligned(16))) uint16_t sB[CH * CH];
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const long long p0 = (long long)xcd_remap(blockIdx.x, gridDim.x) * TP;
  // every load issued before the first wait
  u32x4 rw[8], rg[8], ro[8];
  fetch_block<NT>(rw, a.w_out, CH, tid);
  fetch_block<NT>(rg, a.g + p0 * CH, CH, tid);
  fetch_block<NT>(ro, a.o + p0 * CH, CH, tid);
  put_block<NT>(sB, rw, tid);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int pc = tid + NT * i, row = pc >> 4, c = (pc & 15) * 8;
    float gv[8], ov[8];
    unpack8(rg[i], gv);
    unpack8(ro[i], ov);
#pragma unroll
    for (int e = 0; e < 8; ++e) gv[e] *= ov[e];
    *(u32x4 *)(sA + toff(row, c)) = pack8u(gv);
  }
  __syncthreads();
  const int wm = (wave >> 1) * 64, wn = (wave & 1) * 64;
  f32x16 acc[2][2];
  zero(acc);
  tile_product<ROW, TR>(sA, sB, wm, wn, lane, CH / 16, acc);
  __syncthreads();
  store_tile_bf16(sA, a.y + p0 * CH, acc, wm, wn, lane, tid, [](float x) { return x; });
}

// ------------------------------------------------------------------------------------
// Backward
// ------------------------------------------------------------------------------------
// dgo = dy Wo^T per tile; dO = dgo * g and dgp = dgo * o * g (1 - g), both bf16.
__global__ __launch_bounds__(NT, 2) void mod_out_bwd_kernel(ModArgs a) {
  // the operand tiles, then (after the products) the fp32 tile of dgo in the same space
  __shared__ __attribute__((aligned(16))) float lds[TP * CH];
  uint16_t *sA = (uint16_t *)lds, *sB = sA + TP * CH;
  float *s32 = lds;
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const long long p0 = (long long)xcd_remap(blockIdx.x, gridDim.x) * TP;
  // every load issued at the start: g and o wait in registers for the element-wise step
  u32x4 rd[8], rw[8], rg[8], ro[8];
  fetch_block<NT>(rd, a.dy + p0 * CH, CH, tid);
  fetch_block<NT>(rw, a.w_out, CH, tid);  // Wo [c_in][c_out]: B(t = c_out, n = c_in) as rows
  fetch_block<NT>(rg, a.g + p0 * CH, CH, tid);
  fetch_block<NT>(ro, a.o + p0 * CH, CH, tid);
  put_block<NT>(sA, rd, tid);
  put_block<NT>(sB, rw, tid);
  __syncthreads();
  const int wm = (wave >> 1) * 64, wn = (wave & 1) * 64;
  f32x16 acc[2][2];
  zero(acc);
  tile_product<ROW, ROW>(sA, sB, wm, wn, lane, CH / 16, acc);
  __syncthreads();  // the operand tiles are consumed
  stage_f32(s32, acc, wm, wn, lane, [](float x) { return x; });
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int pc = tid + NT * i, row = pc >> 4, c = (pc & 15) * 8;
    const long long off = (p0 + row) * CH + c;
    float d[8], gv[8], ov[8], dov[8], dgv[8];
    read8_f32(s32, row, c, d);
    unpack8(rg[i], gv);
    unpack8(ro[i], ov);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      dov[e] = d[e] * gv[e];
      dgv[e] = d[e] * ov[e] * gv[e] * (1.f - gv[e]);
    }
    *(u32x4 *)(a.d_o + off) = pack8u(dov);
    *(u32x4 *)(a.dgp + off) = pack8u(dgv);
  }
}

// dzn = [dq dk dv dgp] Wqkvg^T + dbias Wb^T per tile (five contraction blocks of 128,
// the bias block only over its H columns), then the LayerNorm backward
//   dxhat = dzn * w,  dz = rstd (dxhat - mean(dxhat) - xhat mean(dxhat xhat)),
// and the tile's sums over its positions of dzn * xhat and of dzn (partials of the
// LayerNorm scale and offset gradients), each in position order.
// 8 waves (each owning 32 x 64 of dzn), two workgroups per CU: the operand tiles (64 KB)
// are the only large LDS buffer, and once the products are done they hold the fp32 dzn
// tile.  A block's operands are fetched into registers while the previous block's
// products run, z for the LayerNorm backward during the bias block.  The column sums
// recompute xhat from z (read by channel) and the tile's statistics.
__global__ __launch_bounds__(NT8, 4) void mod_in_bwd_kernel(ModArgs a) {
  __shared__ __attribute__((aligned(16))) float lds[TP * CH];  // [sA | sB], then the fp32 dzn tile
  __shared__ f32x2 s_st[TP];
  __shared__ float s_part[2][4][CH];
  uint16_t *sA = (uint16_t *)lds, *sB = sA + TP * CH;
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int tile = xcd_remap(blockIdx.x, gridDim.x);
  const long long p0 = (long long)tile * TP;
  const int wm = (wave >> 1) * 32, wn = (wave & 1) * 64;
  // block blk < 4: A = dq, dk, dv, dgp at the tile's positions, B(t, n = c_in) =
  // Wqkvg[c_in][128 blk + t] (rows)
  auto fetch = [&](int blk, u32x4 (&r)[8]) {
    const uint16_t *src = (blk == 0 ? a.dq : blk == 1 ? a.dk : blk == 2 ? a.dv : a.dgp) + p0 * CH;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int pc = tid + NT8 * i, row = pc >> 4, c = (pc & 15) * 8;
      r[i] = *(const u32x4 *)(src + (long long)row * CH + c);
      r[4 + i] = *(const u32x4 *)(a.w_qkvg + (long long)row * 4 * CH + blk * CH + c);
    }
  };
  auto put = [&](const u32x4 (&r)[8]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int pc = tid + NT8 * i, row = pc >> 4, c = (pc & 15) * 8;
      *(u32x4 *)(sA + toff(row, c)) = r[i];
      *(u32x4 *)(sB + toff(row, c)) = r[4 + i];
    }
  };
  // per position in the LayerNorm backward: thread -> position tid / 4, channels
  // 32 (tid % 4) .. + 31
  const int pr = tid >> 2, c0 = 32 * (tid & 3);
  u32x4 rb[8], zr[4];
  f32x16 acc[1][2];
  zero<1>(acc);
  fetch(0, rb);
#pragma unroll
  for (int blk = 0; blk < 4; ++blk) {
    if (blk) __syncthreads();  // the previous block's operands are consumed
    put(rb);
    __syncthreads();
    if (blk < 3) fetch(blk + 1, rb);
    tile_product_u2<ROW, ROW>(sA, sB, wm, wn, lane, CH / 16, acc);
  }
  // block 4: A(position, t = head) = dbias at that position, rounded to bf16;
  // B(t = head, n = c_in) = Wb[c_in][head]: rows; zeros beyond the H heads.  One 16-deep
  // slice: only columns 0..15 of the two tiles are read.
#pragma unroll
  for (int i = 0; i < 4; ++i) zr[i] = *(const u32x4 *)(a.z + (p0 + pr) * CH + c0 + 8 * i);
  __syncthreads();
  if (tid < 256) {
    const u32x4 z4 = {0u, 0u, 0u, 0u};
    const int row = tid >> 1, c = (tid & 1) * 8;
    *(u32x4 *)(sA + toff(row, c)) = z4;
    *(u32x4 *)(sB + toff(row, c)) = z4;
  }
  if (tid < TP) s_st[tid] = *(const f32x2 *)(a.stats + 2 * (p0 + tid));
  __syncthreads();
  {
    const BiasTile bt(a, p0);
    for (int e = tid; e < TP * a.H; e += NT8) {
      const int row = e / a.H, h = e - row * a.H;
      sA[toff(row, h)] = (uint16_t)(pack_bf16(a.dbias[bt.at(row, h)], 0.f) & 0xffffu);
      sB[toff(row, h)] = a.w_bias[e];  // row = input channel: Wb[c_in][h] is element c_in H + h
    }
  }
  __syncthreads();
  tile_product_u2<ROW, ROW>(sA, sB, wm, wn, lane, 1, acc);
  __syncthreads();  // the operand tiles are consumed
  stage_f32<1>(lds, acc, wm, wn, lane, [](float x) { return x; });
  __syncthreads();
  {
    const f32x2 st = s_st[pr];
    const float mean = st[0], rstd = st[1];
    float s1 = 0.f, s2 = 0.f;
    float dx[32], xh[32];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float zv[8], d[8];
      unpack8(zr[i], zv);
      read8_f32(lds, pr, c0 + 8 * i, d);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int c = 8 * i + e;
        xh[c] = (zv[e] - mean) * rstd;
        dx[c] = d[e] * a.ln_w[c0 + c];
        s1 += dx[c];
        s2 = fmaf(dx[c], xh[c], s2);
      }
    }
    // the four quarters of the position: (q0 + q1) + (q2 + q3) on all four lanes
    s1 += __shfl_xor(s1, 1);
    s2 += __shfl_xor(s2, 1);
    s1 += __shfl_xor(s1, 2);
    s2 += __shfl_xor(s2, 2);
    const float m1 = s1 * (1.f / CH), m2 = s2 * (1.f / CH);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float o[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = rstd * (dx[8 * i + e] - m1 - xh[8 * i + e] * m2);
      *(u32x4 *)(a.dz + (p0 + pr) * CH + c0 + 8 * i) = pack8u(o);
    }
  }
  {
    // column sums: thread -> channel tid % 128, quarter tid / 128 of the positions in
    // order, then the quarters in order; xhat recomputed as in the LayerNorm backward
    const int c = tid & 127, q = tid >> 7;
    float sw = 0.f, sb = 0.f;
#pragma unroll 8
    for (int r = 32 * q; r < 32 * q + 32; ++r) {
      const float d = lds[foff(r, c)];
      const f32x2 st = s_st[r];
      const float xh = (bf_lo(a.z[(p0 + r) * CH + c]) - st[0]) * st[1];
      sw += d * xh;
      sb += d;
    }
    s_part[0][q][c] = sw;
    s_part[1][q][c] = sb;
    __syncthreads();
    if (q == 0) {
      float *part = a.ln_part + (long long)tile * 2 * CH;
      part[c] = ((s_part[0][0][c] + s_part[0][1][c]) + s_part[0][2][c]) + s_part[0][3][c];
      part[CH + c] = ((s_part[1][0][c] + s_part[1][1][c]) + s_part[1][2][c]) + s_part[1][3][c];
    }
  }
}

// Weight gradients: workgroup = (slice of tiles, output block), 8 waves each owning
// 32 x 64 of the 128 x 128 block; out[m][n] = sum over the slice's positions p of
// A[p][m] B[p][n] with
//   blocks 0..3: A = zn, B = dq, dk, dv, dgp      (d Wqkvg, column block 0..3)
//   block 4:     A = zn, B = dbias at p (bf16)    (d Wb, columns < H)
//   block 5:     A = bf16(g * o), B = dy          (d Wo)
// Both operands are read transposed from position-major tiles, fetched into registers a
// tile ahead.  The six blocks of a slice are neighbouring workgroups on one XCD.  The
// fp32 partial of the slice goes to w_part[block][slice].
__global__ __launch_bounds__(NT8, 4) void mod_wgrad_kernel(ModArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t sA[TP * CH];
  __shared__ __attribute__((aligned(16))) uint16_t sB[TP * CH];
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int t = xcd_remap(blockIdx.x, gridDim.x);
  const int blk = t % 6, slice = t / 6;
  const int t0 = (int)((long long)slice * a.tiles / a.slices), t1 = (int)((long long)(slice + 1) * a.tiles / a.slices);
  const int wm = (wave >> 1) * 32, wn = (wave & 1) * 64;
  const uint16_t *asrc = blk < 5 ? a.zn : a.g;
  // the bias block fetches dq as a stand-in B (never used: its B tile is gathered)
  const uint16_t *bsrc = blk == 0 || blk == 4 ? a.dq : blk == 1 ? a.dk : blk == 2 ? a.dv : blk == 3 ? a.dgp : a.dy;
  if (blk == 4) {  // the bias block's B tile: zeros beyond the H head columns
    const u32x4 z4 = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int pc = tid + NT8 * i, row = pc >> 4, c = (pc & 15) * 8;
      *(u32x4 *)(sB + toff(row, c)) = z4;
    }
  }
  u32x4 ra[4], ro[4], rb[4];
  auto fetch = [&](int tile) {
    const long long p0 = (long long)tile * TP;
    fetch_block<NT8>(ra, asrc + p0 * CH, CH, tid);
    fetch_block<NT8>(rb, bsrc + p0 * CH, CH, tid);
    if (blk == 5) fetch_block<NT8>(ro, a.o + p0 * CH, CH, tid);
  };
  f32x16 acc[1][2];
  zero<1>(acc);
  fetch(t0);
#pragma unroll 1
  for (int tile = t0; tile < t1; ++tile) {
    const long long p0 = (long long)tile * TP;
    if (tile > t0) __syncthreads();  // the previous tile's operands are consumed
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int pc = tid + NT8 * i, row = pc >> 4, c = (pc & 15) * 8;
      u32x4 w = ra[i];
      if (blk == 5) {
        float gv[8], ov[8];
        unpack8(ra[i], gv);
        unpack8(ro[i], ov);
#pragma unroll
        for (int e = 0; e < 8; ++e) gv[e] *= ov[e];
        w = pack8u(gv);
      }
      *(u32x4 *)(sA + toff(row, c)) = w;
      if (blk != 4) *(u32x4 *)(sB + toff(row, c)) = rb[i];
    }
    if (blk == 4) {
      // the H head columns of the tile (the others were zeroed before the loop)
      const BiasTile bt(a, p0);
      for (int e = tid; e < TP * a.H; e += NT8) {
        const int row = e / a.H, h = e - row * a.H;
        sB[toff(row, h)] = (uint16_t)(pack_bf16(a.dbias[bt.at(row, h)], 0.f) & 0xffffu);
      }
    }
    __syncthreads();
    fetch(min(tile + 1, t1 - 1));  // in flight during the products (the last tile again at the end)
    tile_product<TR, TR, 1>(sA, sB, wm, wn, lane, TP / 16, acc);
  }
  float *dst = a.w_part + ((long long)blk * a.slices + slice) * CH * CH;
  const int hh = lane >> 5, ll = lane & 31;
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int m = wm + 8 * (r >> 2) + 4 * hh + (r & 3), n = wn + 32 * j + ll;
      dst[m * CH + n] = acc[0][j][r];
    }
}

struct ReduceArgs {
  const float *w_part;
  const float *ln_part;
  float *dw_qkvg, *dw_bias, *dw_out, *d_ln_w, *d_ln_b;
  int H, slices, tiles;
};

// One thread per weight-gradient element: the slices' partials summed in slice order.
__global__ __launch_bounds__(256) void mod_reduce_w_kernel(ReduceArgs a) {
  const int e = blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= 6 * CH * CH) return;
  const int blk = e / (CH * CH), mn = e - blk * CH * CH, m = mn >> 7, n = mn & 127;
  if (blk == 4 && n >= a.H) return;
  const float *src = a.w_part + (long long)blk * a.slices * CH * CH + mn;
  float s = 0.f;
#pragma unroll 8
  for (int sl = 0; sl < a.slices; ++sl) s += src[(long long)sl * CH * CH];
  if (blk < 4) a.dw_qkvg[m * 4 * CH + blk * CH + n] = s;
  else if (blk == 4) a.dw_bias[m * a.H + n] = s;
  else a.dw_out[m * CH + n] = s;
}

// LayerNorm parameter gradients from the per-tile partials part[tile][256] (scale
// gradient in elements 0..127, offset gradient in 128..255) of one or two LayerNorms, in
// two fixed-order stages.  Stage 1, workgroup (group g, LayerNorm l), thread k: the sum
// over the tiles of group g (G contiguous groups) in tile order, to scratch[l][g][k].
__global__ __launch_bounds__(256) void ln_reduce1_kernel(const float *part0, const float *part1, float *scratch,
                                                          int tiles, int groups) {
  const int g = blockIdx.x, l = blockIdx.y, k = threadIdx.x;
  const float *part = l ? part1 : part0;
  const int t0 = (int)((long long)g * tiles / groups), t1 = (int)((long long)(g + 1) * tiles / groups);
  float s = 0.f;
#pragma unroll 8
  for (int t = t0; t < t1; ++t) s += part[(long long)t * 2 * CH + k];
  scratch[((long long)l * groups + g) * 2 * CH + k] = s;
}

// Stage 2, workgroup = 64 of the 256 L outputs, thread (element kk = tid % 64, quarter
// q = tid / 64 of the groups): the quarter's groups in order, then the four quarters in
// order; element k of LayerNorm l to (k < 128 ? w_l : b_l)[k % 128].
__global__ __launch_bounds__(256) void ln_reduce2_kernel(const float *scratch, int groups, float *w0, float *b0,
                                                          float *w1, float *b1) {
  __shared__ float sq[4][64];
  const int kk = threadIdx.x & 63, q = threadIdx.x >> 6;
  const int e = 64 * blockIdx.x + kk, l = e >> 8, k = e & 255;
  const float *src = scratch + (long long)l * groups * 2 * CH + k;
  const int g0 = q * groups / 4, g1 = (q + 1) * groups / 4;
  float s = 0.f;
#pragma unroll 8
  for (int g = g0; g < g1; ++g) s += src[(long long)g * 2 * CH];
  sq[q][kk] = s;
  __syncthreads();
  if (q == 0) {
    const float v = ((sq[0][kk] + sq[1][kk]) + sq[2][kk]) + sq[3][kk];
    float *dst = l ? (k < CH ? w1 : b1) : (k < CH ? w0 : b0);
    dst[k & 127] = v;
  }
}

// Groups of the first stage (a fixed number: results do not depend on the device); its
// scratch, kLnGroups x 256 floats per LayerNorm, is the weight gradients' slice
// partials, already reduced when the stage runs.
constexpr int kLnGroups = 64;

// ------------------------------------------------------------------------------------
// Triangle multiplicative update block around the contraction (tri_mul_module.h)
// ------------------------------------------------------------------------------------
// zn = LayerNorm_in(z); a = sigmoid(zn Wag) (zn Wap) m; b = sigmoid(zn Wbg) (zn Wbp) m;
// g = sigmoid(zn Wg); x = the contraction of a and b (tri_mul_fwd); y = g (LayerNorm_out(x)
// Wo).  a, b, x and their gradients are channel-major [B, C, N, N] (the contraction's
// layout): the 128 positions of a tile are 128 contiguous elements of every channel, so
// such a tile moves as 16-byte rows of a [channel][position] LDS tile, which is also a
// transposed-layout MFMA operand.  A weight block in LDS, [input channel][output
// column], is read transposed by the forward products and as rows by the backward ones.
struct TmbArgs {
  const uint16_t *z;
  const uint8_t *mask;
  const float *ln_in_w, *ln_in_b, *ln_out_w, *ln_out_b;
  const uint16_t *w_in, *w_out;   // [C][5 C], [C][C]
  uint16_t *zn;
  float *stats_in, *stats_out;    // [P][2]
  uint16_t *a, *b;                // channel-major
  uint16_t *g;                    // [P][C]
  const uint16_t *x;              // channel-major
  uint16_t *xn, *y;               // [P][C]
  const uint16_t *dy;
  uint16_t *dyp, *dgp;            // [P][C]: dL/d(xn Wo), the output gate's pre-activation gradient
  uint16_t *dx;                   // channel-major
  const uint16_t *da, *db;        // channel-major
  uint16_t *dag, *dap, *dbg, *dbp;  // channel-major: gradients of the four a / b projections
  uint16_t *dz;
  float *ln_in_part, *ln_out_part, *w_part;
  int B, N;
  long long P, NN;
  int tiles, slices;
  float eps;
};

// the tile's offset in a channel-major tensor: element (channel c, tile position r) is at
// cm + c N^2 + r
__device__ __forceinline__ long long cm_tile(const TmbArgs &a, long long p0) {
  const long long b = p0 / a.NN;
  return b * CH * a.NN + (p0 - b * a.NN);
}
// the [128 channel][128 position] block of a channel-major tensor into an LDS tile, and back
template <int T = NT>
__device__ __forceinline__ void load_cm(uint16_t *tile, const uint16_t *src, long long nn, int tid) {
  load_block<T>(tile, src, nn, tid);
}
template <int T = NT>
__device__ __forceinline__ void store_rows(const uint16_t *tile, uint16_t *dst, long long ld, int tid) {
#pragma unroll
  for (int i = 0; i < 2048 / T; ++i) {
    const int p = tid + T * i, row = p >> 4, c = (p & 15) * 8;
    *(u32x4 *)(dst + (long long)row * ld + c) = *(const u32x4 *)(tile + toff(row, c));
  }
}
__device__ __forceinline__ uint16_t bf16_of(float x) { return (uint16_t)(pack_bf16(x, 0.f) & 0xffffu); }

// LayerNorm of the tile's positions from a position-major bf16 source: thread -> position
// tid / 2, channels 64 (tid % 2) .. + 63; the normalised row goes to tile (row layout)
// and to `out` (bf16), the statistics to `stats`
__device__ __forceinline__ void layer_norm_tile(const uint16_t *src, const float *w, const float *bb, float eps,
                                                uint16_t *tile, uint16_t *out, float *stats, int tid) {
  const int pr = tid >> 1, c0 = 64 * (tid & 1);
  float x[64];
#pragma unroll
  for (int i = 0; i < 8; ++i) unpack8(*(const u32x4 *)(src + pr * CH + c0 + 8 * i), x + 8 * i);
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 64; ++i) s += x[i];
  s += __shfl_xor(s, 1);
  const float mean = s * (1.f / CH);
  float v = 0.f;
#pragma unroll
  for (int i = 0; i < 64; ++i) {
    const float d = x[i] - mean;
    v = fmaf(d, d, v);
  }
  v += __shfl_xor(v, 1);
  const float rstd = 1.f / sqrtf(v * (1.f / CH) + eps);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    float y8[8];
    const f32x4 w0 = *(const f32x4 *)(w + c0 + 8 * i), w1 = *(const f32x4 *)(w + c0 + 8 * i + 4);
    const f32x4 b0 = *(const f32x4 *)(bb + c0 + 8 * i), b1 = *(const f32x4 *)(bb + c0 + 8 * i + 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      y8[e] = fmaf((x[8 * i + e] - mean) * rstd, w0[e], b0[e]);
      y8[4 + e] = fmaf((x[8 * i + 4 + e] - mean) * rstd, w1[e], b1[e]);
    }
    const u32x4 q = pack8u(y8);
    *(u32x4 *)(tile + toff(pr, c0 + 8 * i)) = q;
    *(u32x4 *)(out + pr * CH + c0 + 8 * i) = q;
  }
  if ((tid & 1) == 0) *(f32x2 *)(stats + 2 * pr) = (f32x2){mean, rstd};
}

// Forward, part 1: LayerNorm_in, then the blocks ag, ap (-> a), bg, bp (-> b) and g.
// One workgroup per CU: the gate and projection accumulators of a pair are live at once.
__global__ __launch_bounds__(NT, 1) void tmb_proj_kernel(TmbArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t sA[TP * CH];
  __shared__ __attribute__((aligned(16))) uint16_t sB[CH * CH];
  __shared__ float s_m[TP];
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const long long p0 = (long long)xcd_remap(blockIdx.x, gridDim.x) * TP;
  const long long cm = cm_tile(a, p0);
  u32x4 wr[8];
  auto fetch_w = [&](int blk) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int pc = tid + NT * i, row = pc >> 4, c = (pc & 15) * 8;
      wr[i] = *(const u32x4 *)(a.w_in + (long long)row * 5 * CH + blk * CH + c);
    }
  };
  auto stage_w = [&]() {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int pc = tid + NT * i, row = pc >> 4, c = (pc & 15) * 8;
      *(u32x4 *)(sB + toff(row, c)) = wr[i];
    }
  };
  if (tid < TP) s_m[tid] = a.mask ? (a.mask[p0 + tid] ? 1.f : 0.f) : 1.f;
  fetch_w(0);  // in flight during the LayerNorm
  layer_norm_tile(a.z + p0 * CH, a.ln_in_w, a.ln_in_b, a.eps, sA, a.zn + p0 * CH, a.stats_in + 2 * p0, tid);
  stage_w();
  fetch_w(1);
  __syncthreads();
  const int wm = (wave >> 1) * 64, wn = (wave & 1) * 64, hh = lane >> 5, ll = lane & 31;
  f32x16 acc0[2][2], acc1[2][2];
#pragma unroll 1
  for (int pr = 0; pr < 2; ++pr) {
    zero(acc0);
    tile_product<ROW, TR>(sA, sB, wm, wn, lane, CH / 16, acc0);  // gate pre-activation
    __syncthreads();
    stage_w();
    fetch_w(2 * pr + 2);
    __syncthreads();
    zero(acc1);
    tile_product<ROW, TR>(sA, sB, wm, wn, lane, CH / 16, acc1);  // projection
    __syncthreads();
    // sigmoid(gate) * projection * mask, transposed into [channel][position]
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int m = wm + 32 * i + 8 * (r >> 2) + 4 * hh + (r & 3), n = wn + 32 * j + ll;
          sB[toff(n, m)] = bf16_of(sigmoidf_(acc0[i][j][r]) * acc1[i][j][r] * s_m[m]);
        }
    __syncthreads();
    store_rows(sB, (pr ? a.b : a.a) + cm, a.NN, tid);
    __syncthreads();
    stage_w();
    if (2 * pr + 3 < 5) fetch_w(2 * pr + 3);
    __syncthreads();
  }
  zero(acc0);
  tile_product<ROW, TR>(sA, sB, wm, wn, lane, CH / 16, acc0);
  __syncthreads();
  store_tile_bf16(sB, a.g + p0 * CH, acc0, wm, wn, lane, tid, [](float x) { return sigmoidf_(x); });
}

// Forward, part 2: LayerNorm_out of the contraction's x (read channel-major), then
// y = g * (xn Wo).
__global__ __launch_bounds__(NT, 2) void tmb_out_kernel(TmbArgs a) {
  __shared__ __attribute__((aligned(16))) float lds[TP * CH];  // sA | sB, then the fp32 tile
  uint16_t *sA = (uint16_t *)lds, *sB = sA + TP * CH;
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const long long p0 = (long long)xcd_remap(blockIdx.x, gridDim.x) * TP;
  // every load issued at the start: Wo and g wait in registers
  u32x4 rx[8], rw[8], rg[8];
  fetch_block<NT>(rx, a.x + cm_tile(a, p0), a.NN, tid);  // [channel][position]
  fetch_block<NT>(rw, a.w_out, CH, tid);
  fetch_block<NT>(rg, a.g + p0 * CH, CH, tid);
  put_block<NT>(sB, rx, tid);
  __syncthreads();
  {
    const int pr = tid >> 1, c0 = 64 * (tid & 1);
    float x[64];
#pragma unroll
    for (int i = 0; i < 64; ++i) x[i] = bf_lo(sB[toff(c0 + i, pr)]);
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 64; ++i) s += x[i];
    s += __shfl_xor(s, 1);
    const float mean = s * (1.f / CH);
    float v = 0.f;
#pragma unroll
    for (int i = 0; i < 64; ++i) {
      const float d = x[i] - mean;
      v = fmaf(d, d, v);
    }
    v += __shfl_xor(v, 1);
    const float rstd = 1.f / sqrtf(v * (1.f / CH) + a.eps);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float y8[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) y8[e] = fmaf((x[8 * i + e] - mean) * rstd, a.ln_out_w[c0 + 8 * i + e], a.ln_out_b[c0 + 8 * i + e]);
      const u32x4 q = pack8u(y8);
      *(u32x4 *)(sA + toff(pr, c0 + 8 * i)) = q;
      *(u32x4 *)(a.xn + (p0 + pr) * CH + c0 + 8 * i) = q;
    }
    if ((tid & 1) == 0) *(f32x2 *)(a.stats_out + 2 * (p0 + pr)) = (f32x2){mean, rstd};
  }
  __syncthreads();
  put_block<NT>(sB, rw, tid);
  __syncthreads();
  const int wm = (wave >> 1) * 64, wn = (wave & 1) * 64;
  f32x16 acc[2][2];
  zero(acc);
  tile_product<ROW, TR>(sA, sB, wm, wn, lane, CH / 16, acc);
  __syncthreads();
  stage_f32(lds, acc, wm, wn, lane, [](float x) { return x; });
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int pc = tid + NT * i, row = pc >> 4, c = (pc & 15) * 8;
    const long long off = (p0 + row) * CH + c;
    float yp[8], gv[8];
    read8_f32(lds, row, c, yp);
    unpack8(rg[i], gv);
#pragma unroll
    for (int e = 0; e < 8; ++e) yp[e] *= gv[e];
    *(u32x4 *)(a.y + off) = pack8u(yp);
  }
}

// Backward, part 1: the output gate and projection and LayerNorm_out's backward:
//   yp = xn Wo (recomputed), dyp = dy g, dgp = dy yp g (1 - g), dxn = dyp Wo^T,
//   dx = LayerNorm_out backward of dxn (channel-major), and the tile's column sums of
//   dxn xhat and dxn.
// 8 waves (two per SIMD), each owning 32 x 64 of the products.  Every input of the tile
// (xn, Wo, g, dy and x) is fetched at the start; one Wo tile serves both products
// (transposed reads for yp, row reads for dxn), and the gate's element-wise step runs
// in the accumulator layout against g and dy tiles in LDS, overwriting them in place
// with dgp and dyp.
__global__ __launch_bounds__(NT8, 1) void tmb_out_bwd_kernel(TmbArgs a) {
  __shared__ __attribute__((aligned(16))) float lds[TP * CH];  // xn | g (then dgp), or an fp32 tile
  __shared__ __attribute__((aligned(16))) uint16_t sB[CH * CH];  // Wo
  __shared__ __attribute__((aligned(16))) uint16_t sR[TP * CH];  // dy (then dyp), then x^T (then dx^T)
  __shared__ float s_part[4][CH];
  uint16_t *sA = (uint16_t *)lds, *sG = sA + TP * CH;
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hh = lane >> 5, ll = lane & 31;
  const int tile = xcd_remap(blockIdx.x, gridDim.x);
  const long long p0 = (long long)tile * TP;
  const long long cm = cm_tile(a, p0);
  const int wm = (wave >> 1) * 32, wn = (wave & 1) * 64;
  u32x4 rxn[4], rw[4], rg[4], rdy[4], rx[4];
  fetch_block<NT8>(rxn, a.xn + p0 * CH, CH, tid);
  fetch_block<NT8>(rw, a.w_out, CH, tid);
  fetch_block<NT8>(rg, a.g + p0 * CH, CH, tid);
  fetch_block<NT8>(rdy, a.dy + p0 * CH, CH, tid);
  fetch_block<NT8>(rx, a.x + cm, a.NN, tid);
  put_block<NT8>(sA, rxn, tid);
  put_block<NT8>(sB, rw, tid);
  put_block<NT8>(sG, rg, tid);
  put_block<NT8>(sR, rdy, tid);
  __syncthreads();
  f32x16 acc[1][2];
  zero<1>(acc);
  tile_product<ROW, TR, 1>(sA, sB, wm, wn, lane, CH / 16, acc);  // yp
  // element (m, n) of g and dy is read and overwritten by the lane that holds yp there
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int m = wm + 8 * (r >> 2) + 4 * hh + (r & 3), n = wn + 32 * j + ll;
      const float gv = bf_lo(sG[toff(m, n)]), d = bf_lo(sR[toff(m, n)]);
      sR[toff(m, n)] = bf16_of(d * gv);
      sG[toff(m, n)] = bf16_of(d * acc[0][j][r] * gv * (1.f - gv));
    }
  __syncthreads();
  store_rows<NT8>(sR, a.dyp + p0 * CH, CH, tid);
  store_rows<NT8>(sG, a.dgp + p0 * CH, CH, tid);
  zero<1>(acc);
  tile_product<ROW, ROW, 1>(sR, sB, wm, wn, lane, CH / 16, acc);  // dxn: B(t = c_out, n = c_in) = Wo[c_in][c_out]
  __syncthreads();  // dyp and dgp read; the operand tiles are free
  put_block<NT8>(sR, rx, tid);  // x [channel][position]
  stage_f32<1>(lds, acc, wm, wn, lane, [](float x) { return x; });
  __syncthreads();
  float *part = a.ln_out_part + (long long)tile * 2 * CH;
  column_sums8(lds, s_part, part + CH, tid);  // sum of dxn: the offset gradient's partial
  {
    // thread -> position tid / 4, channels 32 (tid % 4) .. + 31
    const int pr = tid >> 2, c0 = 32 * (tid & 3);
    const f32x2 st = *(const f32x2 *)(a.stats_out + 2 * (p0 + pr));
    const float mean = st[0], rstd = st[1];
    float s1 = 0.f, s2 = 0.f;
    float dx[32], xh[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const int c = c0 + i;
      const float d = lds[foff(pr, c)];
      xh[i] = (bf_lo(sR[toff(c, pr)]) - mean) * rstd;
      dx[i] = d * a.ln_out_w[c];
      s1 += dx[i];
      s2 = fmaf(dx[i], xh[i], s2);
      lds[foff(pr, c)] = d * xh[i];  // dxn * xhat, in place, for the scale gradient
    }
    // the four quarters of the position: (q0 + q1) + (q2 + q3) on all four lanes
    s1 += __shfl_xor(s1, 1);
    s2 += __shfl_xor(s2, 1);
    s1 += __shfl_xor(s1, 2);
    s2 += __shfl_xor(s2, 2);
    const float m1 = s1 * (1.f / CH), m2 = s2 * (1.f / CH);
#pragma unroll
    for (int i = 0; i < 32; ++i) sR[toff(c0 + i, pr)] = bf16_of(rstd * (dx[i] - m1 - xh[i] * m2));
  }
  __syncthreads();
  column_sums8(lds, s_part, part, tid);  // sum of dxn * xhat
  store_rows<NT8>(sR, a.dx + cm, a.NN, tid);
}

// Backward, part 2: the gated projections' gradients from da and db (channel-major),
//   d(ap) = da sigmoid(ag) m,  d(ag) = da ap m sigmoid(ag) (1 - sigmoid(ag))   (b likewise)
// with ag, ap, bg, bp recomputed from zn; stored channel-major.  8 waves, each owning
// 32 x 64 of the products.
__global__ __launch_bounds__(NT8, 1) void tmb_grad_proj_kernel(TmbArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t sA[TP * CH];  // zn
  __shared__ __attribute__((aligned(16))) uint16_t sB[CH * CH];  // weights, then d(proj)
  __shared__ __attribute__((aligned(16))) uint16_t sT[CH * TP];  // da, then d(gate)
  __shared__ float s_m[TP];
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const long long p0 = (long long)xcd_remap(blockIdx.x, gridDim.x) * TP;
  const long long cm = cm_tile(a, p0);
  const int wm = (wave >> 1) * 32, wn = (wave & 1) * 64, hh = lane >> 5, ll = lane & 31;
  if (tid < TP) s_m[tid] = a.mask ? (a.mask[p0 + tid] ? 1.f : 0.f) : 1.f;
  // the operands of pair pr (the gate and projection weight blocks and da or db) are
  // fetched one pair ahead: pair 1's loads are in flight while pair 0 computes
  u32x4 rz[4], rwg[4], rwp[4], rd[4];
  fetch_block<NT8>(rz, a.zn + p0 * CH, CH, tid);
  fetch_block<NT8>(rwg, a.w_in, 5 * CH, tid);
  fetch_block<NT8>(rwp, a.w_in + CH, 5 * CH, tid);
  fetch_block<NT8>(rd, a.da + cm, a.NN, tid);
  put_block<NT8>(sA, rz, tid);
  f32x16 acc_g[1][2], acc_p[1][2];
#pragma unroll
  for (int pr = 0; pr < 2; ++pr) {
    if (pr) __syncthreads();  // the previous pair's results are stored
    put_block<NT8>(sB, rwg, tid);  // the gate block
    __syncthreads();
    zero<1>(acc_g);
    tile_product<ROW, TR, 1>(sA, sB, wm, wn, lane, CH / 16, acc_g);
    __syncthreads();
    put_block<NT8>(sB, rwp, tid);  // the projection block
    put_block<NT8>(sT, rd, tid);
    __syncthreads();
    if (pr == 0) {
      fetch_block<NT8>(rwg, a.w_in + 2 * CH, 5 * CH, tid);
      fetch_block<NT8>(rwp, a.w_in + 3 * CH, 5 * CH, tid);
      fetch_block<NT8>(rd, a.db + cm, a.NN, tid);
    }
    zero<1>(acc_p);
    tile_product<ROW, TR, 1>(sA, sB, wm, wn, lane, CH / 16, acc_p);
    __syncthreads();  // sB is free for d(proj)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = wm + 8 * (r >> 2) + 4 * hh + (r & 3), n = wn + 32 * j + ll;
        const float d = bf_lo(sT[toff(n, m)]) * s_m[m];
        const float sg = sigmoidf_(acc_g[0][j][r]);
        sT[toff(n, m)] = bf16_of(d * acc_p[0][j][r] * sg * (1.f - sg));
        sB[toff(n, m)] = bf16_of(d * sg);
      }
    __syncthreads();
    store_rows<NT8>(sT, (pr ? a.dbg : a.dag) + cm, a.NN, tid);
    store_rows<NT8>(sB, (pr ? a.dbp : a.dap) + cm, a.NN, tid);
  }
}

// Backward, part 3: dzn = [d(ag) d(ap) d(bg) d(bp) dgp] Win^T (five 128-deep blocks), the
// LayerNorm_in backward to dz and the tile's column sums of dzn xhat and dzn.
// 8 waves (each owning 32 x 64 of dzn), two workgroups per CU: the operand tiles (64 KB)
// are the only large LDS buffer, and once the products are done they hold the fp32 dzn
// tile.  A block's operands are fetched into registers while the previous block's
// products run, z for the LayerNorm backward during the last one's.  The column sums
// recompute xhat from z (read by channel) and the tile's statistics.
__global__ __launch_bounds__(NT8, 4) void tmb_in_bwd_kernel(TmbArgs a) {
  __shared__ __attribute__((aligned(16))) float lds[TP * CH];  // [sA | sB], then the fp32 dzn tile
  __shared__ f32x2 s_st[TP];
  __shared__ float s_part[2][4][CH];
  uint16_t *sA = (uint16_t *)lds, *sB = sA + TP * CH;
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int tile = xcd_remap(blockIdx.x, gridDim.x);
  const long long p0 = (long long)tile * TP;
  const long long cm = cm_tile(a, p0);
  const int wm = (wave >> 1) * 32, wn = (wave & 1) * 64;
  // block blk: A = d(ag), d(ap), d(bg), d(bp) ([channel][position], read transposed) or
  // dgp ([position][channel]); B(t = out, n = c_in) = Win[c_in][128 blk + t] (rows)
  auto fetch = [&](int blk, u32x4 (&r)[8]) {
    const uint16_t *src = blk == 0 ? a.dag + cm : blk == 1 ? a.dap + cm : blk == 2 ? a.dbg + cm
                        : blk == 3 ? a.dbp + cm : a.dgp + p0 * CH;
    const long long ld = blk < 4 ? a.NN : CH;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int pc = tid + NT8 * i, row = pc >> 4, c = (pc & 15) * 8;
      r[i] = *(const u32x4 *)(src + (long long)row * ld + c);
      r[4 + i] = *(const u32x4 *)(a.w_in + (long long)row * 5 * CH + blk * CH + c);
    }
  };
  auto put = [&](const u32x4 (&r)[8]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int pc = tid + NT8 * i, row = pc >> 4, c = (pc & 15) * 8;
      *(u32x4 *)(sA + toff(row, c)) = r[i];
      *(u32x4 *)(sB + toff(row, c)) = r[4 + i];
    }
  };
  // per position in the LayerNorm backward: thread -> position tid / 4, channels
  // 32 (tid % 4) .. + 31
  const int pr = tid >> 2, c0 = 32 * (tid & 3);
  u32x4 rb[8], zr[4];
  f32x16 dzn[1][2];
  zero<1>(dzn);
  fetch(0, rb);
#pragma unroll
  for (int blk = 0; blk < 5; ++blk) {
    if (blk) __syncthreads();  // the previous block's operands are consumed
    put(rb);
    __syncthreads();
    if (blk < 4) {
      fetch(blk + 1, rb);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) zr[i] = *(const u32x4 *)(a.z + (p0 + pr) * CH + c0 + 8 * i);
    }
    if (blk < 4) tile_product_u2<TR, ROW>(sA, sB, wm, wn, lane, CH / 16, dzn);
    else tile_product_u2<ROW, ROW>(sA, sB, wm, wn, lane, CH / 16, dzn);
  }
  if (tid < TP) s_st[tid] = *(const f32x2 *)(a.stats_in + 2 * (p0 + tid));
  __syncthreads();  // the operand tiles are consumed
  stage_f32<1>(lds, dzn, wm, wn, lane, [](float x) { return x; });
  __syncthreads();
  {
    const f32x2 st = s_st[pr];
    const float mean = st[0], rstd = st[1];
    float s1 = 0.f, s2 = 0.f;
    float dx[32], xh[32];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float zv[8], d[8];
      unpack8(zr[i], zv);
      read8_f32(lds, pr, c0 + 8 * i, d);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int c = 8 * i + e;
        xh[c] = (zv[e] - mean) * rstd;
        dx[c] = d[e] * a.ln_in_w[c0 + c];
        s1 += dx[c];
        s2 = fmaf(dx[c], xh[c], s2);
      }
    }
    // the four quarters of the position: (q0 + q1) + (q2 + q3) on all four lanes
    s1 += __shfl_xor(s1, 1);
    s2 += __shfl_xor(s2, 1);
    s1 += __shfl_xor(s1, 2);
    s2 += __shfl_xor(s2, 2);
    const float m1 = s1 * (1.f / CH), m2 = s2 * (1.f / CH);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float o[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = rstd * (dx[8 * i + e] - m1 - xh[8 * i + e] * m2);
      *(u32x4 *)(a.dz + (p0 + pr) * CH + c0 + 8 * i) = pack8u(o);
    }
  }
  {
    // column sums: thread -> channel tid % 128, quarter tid / 128 of the positions in
    // order, then the quarters in order; xhat recomputed as in the LayerNorm backward
    const int c = tid & 127, q = tid >> 7;
    float sw = 0.f, sb = 0.f;
#pragma unroll 8
    for (int r = 32 * q; r < 32 * q + 32; ++r) {
      const float d = lds[foff(r, c)];
      const f32x2 st = s_st[r];
      const float xh = (bf_lo(a.z[(p0 + r) * CH + c]) - st[0]) * st[1];
      sw += d * xh;
      sb += d;
    }
    s_part[0][q][c] = sw;
    s_part[1][q][c] = sb;
    __syncthreads();
    if (q == 0) {
      float *part = a.ln_in_part + (long long)tile * 2 * CH;
      part[c] = ((s_part[0][0][c] + s_part[0][1][c]) + s_part[0][2][c]) + s_part[0][3][c];
      part[CH + c] = ((s_part[1][0][c] + s_part[1][1][c]) + s_part[1][2][c]) + s_part[1][3][c];
    }
  }
}

// Weight gradients of the block: workgroup = (slice of tiles, output block), 8 waves
// each owning 32 x 64 of the 128 x 128 block; out[m][n] = sum over the slice's positions
// p of A[p][m] B[p][n] with
//   blocks 0..3: A = zn, B = d(ag), d(ap), d(bg), d(bp)   (B channel-major)
//   block 4:     A = zn, B = dgp
//   block 5:     A = xn, B = dyp                           (d Wo)
// A tile's operands are fetched into registers a tile ahead.  The six blocks of a slice
// are neighbouring workgroups on one XCD, so each zn tile comes from HBM about once.
__global__ __launch_bounds__(NT8, 4) void tmb_wgrad_kernel(TmbArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t sA[TP * CH];
  __shared__ __attribute__((aligned(16))) uint16_t sB[TP * CH];
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int t = xcd_remap(blockIdx.x, gridDim.x);
  const int blk = t % 6, slice = t / 6;
  const int t0 = (int)((long long)slice * a.tiles / a.slices), t1 = (int)((long long)(slice + 1) * a.tiles / a.slices);
  const int wm = (wave >> 1) * 32, wn = (wave & 1) * 64;
  const uint16_t *asrc = blk < 5 ? a.zn : a.xn;
  const uint16_t *bsrc = blk == 0 ? a.dag : blk == 1 ? a.dap : blk == 2 ? a.dbg : blk == 3 ? a.dbp
                       : blk == 4 ? a.dgp : a.dyp;
  f32x16 acc[1][2];
  zero<1>(acc);
  // one copy of the loop per B layout: [channel n][position t] (CMB) or [position t][channel n]
  auto run = [&](auto cmb_tag) {
    constexpr bool CMB = decltype(cmb_tag)::value;
    u32x4 ra[4], rb[4];
    auto fetch = [&](int tile) {
      const long long p0 = (long long)tile * TP;
      fetch_block<NT8>(ra, asrc + p0 * CH, CH, tid);
      if (CMB) fetch_block<NT8>(rb, bsrc + cm_tile(a, p0), a.NN, tid);
      else fetch_block<NT8>(rb, bsrc + p0 * CH, CH, tid);
    };
    fetch(t0);
#pragma unroll 1
    for (int tile = t0; tile < t1; ++tile) {
      if (tile > t0) __syncthreads();  // the previous tile's operands are consumed
      put_block<NT8>(sA, ra, tid);
      put_block<NT8>(sB, rb, tid);
      __syncthreads();
      fetch(min(tile + 1, t1 - 1));  // in flight during the products (the last tile again at the end)
      tile_product<TR, CMB ? ROW : TR, 1>(sA, sB, wm, wn, lane, TP / 16, acc);
    }
  };
  if (blk < 4) run(std::true_type{});
  else run(std::false_type{});
  float *dst = a.w_part + ((long long)blk * a.slices + slice) * CH * CH;
  const int hh = lane >> 5, ll = lane & 31;
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int m = wm + 8 * (r >> 2) + 4 * hh + (r & 3), n = wn + 32 * j + ll;
      dst[m * CH + n] = acc[0][j][r];
    }
}

struct TmbReduceArgs {
  const float *w_part, *ln_in_part, *ln_out_part;
  float *dw_in, *dw_out, *d_ln_in_w, *d_ln_in_b, *d_ln_out_w, *d_ln_out_b;
  int slices, tiles;
};

__global__ __launch_bounds__(256) void tmb_reduce_w_kernel(TmbReduceArgs a) {
  const int e = blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= 6 * CH * CH) return;
  const int blk = e / (CH * CH), mn = e - blk * CH * CH, m = mn >> 7, n = mn & 127;
  const float *src = a.w_part + (long long)blk * a.slices * CH * CH + mn;
  float s = 0.f;
#pragma unroll 8
  for (int sl = 0; sl < a.slices; ++sl) s += src[(long long)sl * CH * CH];
  if (blk < 5) a.dw_in[m * 5 * CH + blk * CH + n] = s;
  else a.dw_out[m * CH + n] = s;
}

// ------------------------------------------------------------------------------------
// Host side
// ------------------------------------------------------------------------------------
constexpr size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

bool aligned16(const void *p) { return p && ((uintptr_t)p & 15u) == 0; }

// Byte ranges of the tensors of a call: every output must be disjoint from every input
// and from every other output.
struct Span {
  uintptr_t lo, hi;
};
Span span(const void *p, size_t bytes) { return {(uintptr_t)p, (uintptr_t)p + (p ? bytes : 0)}; }
bool overlap(Span x, Span y) { return x.lo < y.hi && y.lo < x.hi; }
template <size_t NO, size_t NI>
bool outputs_disjoint(const Span (&outs)[NO], const Span (&ins)[NI]) {
  for (size_t i = 0; i < NO; ++i) {
    for (size_t j = 0; j < NI; ++j)
      if (overlap(outs[i], ins[j])) return false;
    for (size_t k = 0; k < NO; ++k)
      if (k != i && overlap(outs[i], outs[k])) return false;
  }
  return true;
}

tri_attn_status check(const tri_attn_module_problem *p) {
  if (!p) return TRI_ATTN_ERROR_INVALID_VALUE;
  if (p->abi_version != TRI_ATTN_MODULE_ABI_VERSION) return TRI_ATTN_ERROR_ABI_MISMATCH;
  if (p->B < 1 || p->N < 1 || p->H < 1 || p->D < 1) return TRI_ATTN_ERROR_INVALID_VALUE;
  if (!(p->ln_eps >= 0.f) || isinf(p->ln_eps)) return TRI_ATTN_ERROR_INVALID_VALUE;
  if (p->flags & ~TRI_ATTN_FLAG_ENDING_NODE) return TRI_ATTN_ERROR_NOT_SUPPORTED;
  if (p->H * p->D != CH) return TRI_ATTN_ERROR_NOT_SUPPORTED;
  return TRI_ATTN_SUCCESS;  // N, H and D are further checked by the core's validation
}

tri_attn_problem core_problem(const tri_attn_module_problem *p) {
  tri_attn_problem c;
  memset(&c, 0, sizeof c);
  c.abi_version = TRI_ATTN_ABI_VERSION;
  c.flags = (p->flags & TRI_ATTN_FLAG_ENDING_NODE) ? TRI_ATTN_FLAG_ENDING_NODE : 0;
  c.B = p->B;
  c.N = p->N;
  c.H = p->H;
  c.D = p->D;
  c.softmax_scale = 0.f;
  return c;
}

ModArgs base_args(const tri_attn_module_problem *p) {
  ModArgs a;
  memset(&a, 0, sizeof a);
  a.B = (int)p->B;
  a.N = (int)p->N;
  a.H = (int)p->H;
  a.ending = (p->flags & TRI_ATTN_FLAG_ENDING_NODE) ? 1 : 0;
  a.P = p->B * p->N * p->N;
  a.tiles = (int)(a.P / TP);
  a.eps = p->ln_eps > 0.f ? p->ln_eps : 1e-5f;
  return a;
}

// Slices of the weight gradients: 6 x 85 = 510 workgroups, one round at two 8-wave
// workgroups per CU on a 256-CU device (a fixed number, so results do not depend on the
// device).
int wgrad_slices(int tiles) { return tiles < 85 ? tiles : 85; }

struct BwdLayout {
  size_t off_do, off_dgp, off_dq, off_dk, off_dv, off_db, off_core, off_w, off_ln, total;
  size_t core_bytes;
  int slices;
};

BwdLayout bwd_layout(const tri_attn_module_problem *p, size_t core_bytes) {
  BwdLayout l;
  const size_t E = (size_t)p->B * p->N * p->N * CH * 2;  // one bf16 position tensor
  const int tiles = (int)(p->B * p->N * p->N / TP);
  l.slices = wgrad_slices(tiles);
  l.core_bytes = core_bytes;
  size_t o = 0;
  l.off_do = o; o += align256(E);
  l.off_dgp = o; o += align256(E);
  l.off_dq = o; o += align256(E);
  l.off_dk = o; o += align256(E);
  l.off_dv = o; o += align256(E);
  l.off_db = o; o += align256((size_t)p->B * p->H * p->N * p->N * 4);
  l.off_core = o; o += align256(core_bytes);
  l.off_w = o; o += align256((size_t)6 * l.slices * CH * CH * 4);
  l.off_ln = o; o += align256((size_t)tiles * 2 * CH * 4);
  l.total = o;
  return l;
}

tri_attn_status tmb_check(const tri_mul_module_problem *p) {
  if (!p) return TRI_ATTN_ERROR_INVALID_VALUE;
  if (p->abi_version != TRI_MUL_MODULE_ABI_VERSION) return TRI_ATTN_ERROR_ABI_MISMATCH;
  if (p->B < 1 || p->N < 1 || p->C < 1) return TRI_ATTN_ERROR_INVALID_VALUE;
  if (!(p->ln_eps >= 0.f) || isinf(p->ln_eps)) return TRI_ATTN_ERROR_INVALID_VALUE;
  if (p->flags & ~TRI_MUL_FLAG_INCOMING) return TRI_ATTN_ERROR_NOT_SUPPORTED;
  if (p->C != CH || p->N % 32 != 0 || p->N > 1024 || p->B * p->C > 65536) return TRI_ATTN_ERROR_NOT_SUPPORTED;
  return TRI_ATTN_SUCCESS;
}

tri_mul_problem tmb_contraction(const tri_mul_module_problem *p) {
  tri_mul_problem m;
  memset(&m, 0, sizeof m);
  m.abi_version = TRI_MUL_ABI_VERSION;
  m.flags = p->flags & TRI_MUL_FLAG_INCOMING;
  m.B = p->B;
  m.N = p->N;
  m.C = p->C;
  return m;
}

TmbArgs tmb_args(const tri_mul_module_problem *p, const void *z, const uint8_t *mask,
                 const tri_mul_module_params *pr, const tri_mul_module_saved *sv) {
  TmbArgs a;
  memset(&a, 0, sizeof a);
  a.z = (const uint16_t *)z;
  a.mask = mask;
  a.ln_in_w = pr->ln_in_w;
  a.ln_in_b = pr->ln_in_b;
  a.ln_out_w = pr->ln_out_w;
  a.ln_out_b = pr->ln_out_b;
  a.w_in = (const uint16_t *)pr->w_in;
  a.w_out = (const uint16_t *)pr->w_out;
  a.zn = (uint16_t *)sv->zn;
  a.stats_in = sv->ln_in_stats;
  a.stats_out = sv->ln_out_stats;
  a.a = (uint16_t *)sv->a;
  a.b = (uint16_t *)sv->b;
  a.g = (uint16_t *)sv->g;
  a.x = (const uint16_t *)sv->x;
  a.xn = (uint16_t *)sv->xn;
  a.B = (int)p->B;
  a.N = (int)p->N;
  a.NN = p->N * p->N;
  a.P = p->B * a.NN;
  a.tiles = (int)(a.P / TP);
  a.slices = wgrad_slices(a.tiles);
  a.eps = p->ln_eps > 0.f ? p->ln_eps : 1e-5f;
  return a;
}

struct TmbLayout {
  size_t off_dyp, off_dgp, off_dx, off_da, off_db, off_dag, off_dap, off_dbg, off_dbp, off_w, off_lni, off_lno, total;
};

TmbLayout tmb_layout(const tri_mul_module_problem *p) {
  TmbLayout l;
  const size_t E = (size_t)p->B * p->N * p->N * CH * 2;
  const int tiles = (int)(p->B * p->N * p->N / TP);
  size_t o = 0;
  size_t *bf[] = {&l.off_dyp, &l.off_dgp, &l.off_dx, &l.off_da, &l.off_db, &l.off_dag, &l.off_dap, &l.off_dbg,
                  &l.off_dbp};
  for (size_t *x : bf) {
    *x = o;
    o += align256(E);
  }
  l.off_w = o; o += align256((size_t)6 * wgrad_slices(tiles) * CH * CH * 4);
  l.off_lni = o; o += align256((size_t)tiles * 2 * CH * 4);
  l.off_lno = o; o += align256((size_t)tiles * 2 * CH * 4);
  l.total = o;
  return l;
}

}  // namespace

extern "C" {

int tri_mul_module_abi_version(void) { return TRI_MUL_MODULE_ABI_VERSION; }

tri_attn_status tri_mul_module_fwd(const tri_mul_module_problem *problem, const void *z, const uint8_t *mask,
                                   const tri_mul_module_params *params, void *y, const tri_mul_module_saved *saved,
                                   hipStream_t stream) {
  tri_attn_status st = tmb_check(problem);
  if (st != TRI_ATTN_SUCCESS) return st;
  if (!params || !saved) return TRI_ATTN_ERROR_INVALID_VALUE;
  const void *need[] = {z, y, params->ln_in_w, params->ln_in_b, params->w_in, params->ln_out_w, params->ln_out_b,
                        params->w_out, saved->zn, saved->ln_in_stats, saved->a, saved->b, saved->g, saved->x,
                        saved->xn, saved->ln_out_stats};
  for (const void *x : need)
    if (!aligned16(x)) return TRI_ATTN_ERROR_INVALID_VALUE;
  {
    const size_t P = (size_t)problem->B * problem->N * problem->N, E = P * CH * 2;
    const Span ins[] = {span(z, E), span(mask, mask ? P : 0), span(params->ln_in_w, CH * 4),
                        span(params->ln_in_b, CH * 4), span(params->w_in, CH * 5 * CH * 2),
                        span(params->ln_out_w, CH * 4), span(params->ln_out_b, CH * 4),
                        span(params->w_out, CH * CH * 2)};
    const Span outs[] = {span(y, E), span(saved->zn, E), span(saved->ln_in_stats, P * 8), span(saved->a, E),
                         span(saved->b, E), span(saved->g, E), span(saved->x, E), span(saved->xn, E),
                         span(saved->ln_out_stats, P * 8)};
    if (!outputs_disjoint(outs, ins)) return TRI_ATTN_ERROR_INVALID_VALUE;
  }
  TmbArgs a = tmb_args(problem, z, mask, params, saved);
  a.y = (uint16_t *)y;
  hipLaunchKernelGGL(tmb_proj_kernel, dim3((unsigned)a.tiles), dim3(NT), 0, stream, a);
  if (hipGetLastError() != hipSuccess) return TRI_ATTN_ERROR_LAUNCH_FAILED;
  const tri_mul_problem mp = tmb_contraction(problem);
  st = tri_mul_fwd(&mp, saved->a, saved->b, saved->x, stream);
  if (st != TRI_ATTN_SUCCESS) return st;
  hipLaunchKernelGGL(tmb_out_kernel, dim3((unsigned)a.tiles), dim3(NT), 0, stream, a);
  return hipGetLastError() == hipSuccess ? TRI_ATTN_SUCCESS : TRI_ATTN_ERROR_LAUNCH_FAILED;
}

size_t tri_mul_module_bwd_workspace_bytes(const tri_mul_module_problem *problem) {
  if (tmb_check(problem) != TRI_ATTN_SUCCESS) return 0;
  return tmb_layout(problem).total;
}

tri_attn_status tri_mul_module_bwd(const tri_mul_module_problem *problem, const void *z, const uint8_t *mask,
                                   const tri_mul_module_params *params, const tri_mul_module_saved *saved,
                                   const void *dy, void *dz, const tri_mul_module_param_grads *grads,
                                   void *workspace, size_t workspace_bytes, hipStream_t stream) {
  tri_attn_status st = tmb_check(problem);
  if (st != TRI_ATTN_SUCCESS) return st;
  if (!params || !saved || !grads) return TRI_ATTN_ERROR_INVALID_VALUE;
  const void *need[] = {z, dy, dz, params->ln_in_w, params->ln_in_b, params->w_in, params->ln_out_w,
                        params->ln_out_b, params->w_out, saved->zn, saved->ln_in_stats, saved->a, saved->b, saved->g,
                        saved->x, saved->xn, saved->ln_out_stats, grads->ln_in_w, grads->ln_in_b, grads->w_in,
                        grads->ln_out_w, grads->ln_out_b, grads->w_out};
  for (const void *x : need)
    if (!aligned16(x)) return TRI_ATTN_ERROR_INVALID_VALUE;
  if (!workspace || ((uintptr_t)workspace & 255u)) return TRI_ATTN_ERROR_INVALID_VALUE;
  const TmbLayout l = tmb_layout(problem);
  if (workspace_bytes < l.total) return TRI_ATTN_ERROR_INSUFFICIENT_WORKSPACE;
  {
    const size_t P = (size_t)problem->B * problem->N * problem->N, E = P * CH * 2;
    const Span ins[] = {span(z, E), span(mask, mask ? P : 0), span(dy, E), span(params->ln_in_w, CH * 4),
                        span(params->ln_in_b, CH * 4), span(params->w_in, CH * 5 * CH * 2),
                        span(params->ln_out_w, CH * 4), span(params->ln_out_b, CH * 4),
                        span(params->w_out, CH * CH * 2), span(saved->zn, E), span(saved->ln_in_stats, P * 8),
                        span(saved->a, E), span(saved->b, E), span(saved->g, E), span(saved->x, E),
                        span(saved->xn, E), span(saved->ln_out_stats, P * 8)};
    const Span outs[] = {span(dz, E), span(grads->ln_in_w, CH * 4), span(grads->ln_in_b, CH * 4),
                         span(grads->w_in, CH * 5 * CH * 4), span(grads->ln_out_w, CH * 4),
                         span(grads->ln_out_b, CH * 4), span(grads->w_out, CH * CH * 4), span(workspace, l.total)};
    if (!outputs_disjoint(outs, ins)) return TRI_ATTN_ERROR_INVALID_VALUE;
  }
  char *ws = (char *)workspace;
  TmbArgs a = tmb_args(problem, z, mask, params, saved);
  a.dy = (const uint16_t *)dy;
  a.dyp = (uint16_t *)(ws + l.off_dyp);
  a.dgp = (uint16_t *)(ws + l.off_dgp);
  a.dx = (uint16_t *)(ws + l.off_dx);
  a.da = (const uint16_t *)(ws + l.off_da);
  a.db = (const uint16_t *)(ws + l.off_db);
  a.dag = (uint16_t *)(ws + l.off_dag);
  a.dap = (uint16_t *)(ws + l.off_dap);
  a.dbg = (uint16_t *)(ws + l.off_dbg);
  a.dbp = (uint16_t *)(ws + l.off_dbp);
  a.dz = (uint16_t *)dz;
  a.w_part = (float *)(ws + l.off_w);
  a.ln_in_part = (float *)(ws + l.off_lni);
  a.ln_out_part = (float *)(ws + l.off_lno);
  hipLaunchKernelGGL(tmb_out_bwd_kernel, dim3((unsigned)a.tiles), dim3(NT8), 0, stream, a);
  if (hipGetLastError() != hipSuccess) return TRI_ATTN_ERROR_LAUNCH_FAILED;
  const tri_mul_problem mp = tmb_contraction(problem);
  st = tri_mul_bwd(&mp, saved->a, saved->b, a.dx, ws + l.off_da, ws + l.off_db, stream);
  if (st != TRI_ATTN_SUCCESS) return st;
  hipLaunchKernelGGL(tmb_grad_proj_kernel, dim3((unsigned)a.tiles), dim3(NT8), 0, stream, a);
  if (hipGetLastError() != hipSuccess) return TRI_ATTN_ERROR_LAUNCH_FAILED;
  hipLaunchKernelGGL(tmb_in_bwd_kernel, dim3((unsigned)a.tiles), dim3(NT8), 0, stream, a);
  if (hipGetLastError() != hipSuccess) return TRI_ATTN_ERROR_LAUNCH_FAILED;
  hipLaunchKernelGGL(tmb_wgrad_kernel, dim3((unsigned)(6 * a.slices)), dim3(NT8), 0, stream, a);
  if (hipGetLastError() != hipSuccess) return TRI_ATTN_ERROR_LAUNCH_FAILED;
  TmbReduceArgs r;
  r.w_part = a.w_part;
  r.ln_in_part = a.ln_in_part;
  r.ln_out_part = a.ln_out_part;
  r.dw_in = grads->w_in;
  r.dw_out = grads->w_out;
  r.d_ln_in_w = grads->ln_in_w;
  r.d_ln_in_b = grads->ln_in_b;
  r.d_ln_out_w = grads->ln_out_w;
  r.d_ln_out_b = grads->ln_out_b;
  r.slices = a.slices;
  r.tiles = a.tiles;
  hipLaunchKernelGGL(tmb_reduce_w_kernel, dim3((6 * CH * CH + 255) / 256), dim3(256), 0, stream, r);
  if (hipGetLastError() != hipSuccess) return TRI_ATTN_ERROR_LAUNCH_FAILED;
  hipLaunchKernelGGL(ln_reduce1_kernel, dim3(kLnGroups, 2), dim3(256), 0, stream, r.ln_in_part, r.ln_out_part,
                     a.w_part, a.tiles, kLnGroups);
  if (hipGetLastError() != hipSuccess) return TRI_ATTN_ERROR_LAUNCH_FAILED;
  hipLaunchKernelGGL(ln_reduce2_kernel, dim3(8), dim3(256), 0, stream, (const float *)a.w_part, kLnGroups,
                     r.d_ln_in_w, r.d_ln_in_b, r.d_ln_out_w, r.d_ln_out_b);
  return hipGetLastError() == hipSuccess ? TRI_ATTN_SUCCESS : TRI_ATTN_ERROR_LAUNCH_FAILED;
}

int tri_attn_module_abi_version(void) { return TRI_ATTN_MODULE_ABI_VERSION; }

tri_attn_status tri_attn_module_fwd(const tri_attn_module_problem *problem, const void *z, const uint8_t *mask,
                                    const tri_attn_module_params *params, void *y,
                                    const tri_attn_module_saved *saved, hipStream_t stream) {
  tri_attn_status st = check(problem);
  if (st != TRI_ATTN_SUCCESS) return st;
  const tri_attn_problem cp = core_problem(problem);
  // the core's own validation (sizes) before anything is enqueued
  if (tri_attn_bwd_workspace_bytes(&cp) == 0) return TRI_ATTN_ERROR_NOT_SUPPORTED;
  if (!params || !saved) return TRI_ATTN_ERROR_INVALID_VALUE;
  const void *need[] = {z, y, params->ln_w, params->ln_b, params->w_qkvg, params->w_bias, params->w_out,
                        saved->zn, saved->ln_stats, saved->q, saved->k, saved->v, saved->g, saved->bias,
                        saved->o, saved->o_residual, saved->lse};
  for (const void *x : need)
    if (!aligned16(x)) return TRI_ATTN_ERROR_INVALID_VALUE;
  const size_t P = (size_t)problem->B * problem->N * problem->N, E = P * CH * 2;
  const size_t nb = (size_t)problem->B * problem->H * problem->N * problem->N;
  const Span ins[] = {span(z, E), span(mask, mask ? P : 0), span(params->ln_w, CH * 4), span(params->ln_b, CH * 4),
                      span(params->w_qkvg, CH * 4 * CH * 2), span(params->w_bias, CH * problem->H * 2),
                      span(params->w_out, CH * CH * 2)};
  const Span outs[] = {span(y, E), span(saved->zn, E), span(saved->ln_stats, P * 8), span(saved->q, E),
                       span(saved->k, E), span(saved->v, E), span(saved->g, E), span(saved->bias, nb * 2),
                       span(saved->o, E), span(saved->o_residual, 2 * E),
                       span(saved->lse, (size_t)problem->B * problem->N * problem->H * problem->N * 4)};
  if (!outputs_disjoint(outs, ins)) return TRI_ATTN_ERROR_INVALID_VALUE;
  ModArgs a = base_args(problem);
  a.z = (const uint16_t *)z;
  a.ln_w = params->ln_w;
  a.ln_b = params->ln_b;
  a.w_qkvg = (const uint16_t *)params->w_qkvg;
  a.w_bias = (const uint16_t *)params->w_bias;
  a.w_out = (const uint16_t *)params->w_out;
  a.zn = (uint16_t *)saved->zn;
  a.stats = saved->ln_stats;
  a.q = (uint16_t *)saved->q;
  a.k = (uint16_t *)saved->k;
  a.v = (uint16_t *)saved->v;
  a.g = (uint16_t *)saved->g;
  a.bias = (uint16_t *)saved->bias;
  a.o = (uint16_t *)saved->o;
  a.y = (uint16_t *)y;
  hipLaunchKernelGGL(mod_proj_kernel, dim3((unsigned)a.tiles), dim3(NT), 0, stream, a);
  if (hipGetLastError() != hipSuccess) return TRI_ATTN_ERROR_LAUNCH_FAILED;
  st = tri_attn_fwd(&cp, saved->q, saved->k, saved->v, saved->bias, mask, saved->o, saved->o_residual, saved->lse,
                    stream);
  if (st != TRI_ATTN_SUCCESS) return st;
  hipLaunchKernelGGL(mod_gate_out_kernel, dim3((unsigned)a.tiles), dim3(NT), 0, stream, a);
  return hipGetLastError() == hipSuccess ? TRI_ATTN_SUCCESS : TRI_ATTN_ERROR_LAUNCH_FAILED;
}

size_t tri_attn_module_bwd_workspace_bytes(const tri_attn_module_problem *problem) {
  if (check(problem) != TRI_ATTN_SUCCESS) return 0;
  const tri_attn_problem cp = core_problem(problem);
  const size_t core = tri_attn_bwd_workspace_bytes(&cp);
  if (core == 0) return 0;
  return bwd_layout(problem, core).total;
}

tri_attn_status tri_attn_module_bwd(const tri_attn_module_problem *problem, const void *z, const uint8_t *mask,
                                    const tri_attn_module_params *params, const tri_attn_module_saved *saved,
                                    const void *dy, void *dz, const tri_attn_module_param_grads *grads,
                                    void *workspace, size_t workspace_bytes, hipStream_t stream) {
  tri_attn_status st = check(problem);
  if (st != TRI_ATTN_SUCCESS) return st;
  const tri_attn_problem cp = core_problem(problem);
  const size_t core = tri_attn_bwd_workspace_bytes(&cp);
  if (core == 0) return TRI_ATTN_ERROR_NOT_SUPPORTED;
  if (!params || !saved || !grads) return TRI_ATTN_ERROR_INVALID_VALUE;
  const void *need[] = {z, dy, dz, params->ln_w, params->ln_b, params->w_qkvg, params->w_bias, params->w_out,
                        saved->zn, saved->ln_stats, saved->q, saved->k, saved->v, saved->g, saved->bias, saved->o,
                        saved->o_residual, saved->lse, grads->ln_w, grads->ln_b, grads->w_qkvg, grads->w_bias,
                        grads->w_out};
  for (const void *x : need)
    if (!aligned16(x)) return TRI_ATTN_ERROR_INVALID_VALUE;
  if (!workspace || ((uintptr_t)workspace & 255u)) return TRI_ATTN_ERROR_INVALID_VALUE;
  const BwdLayout l = bwd_layout(problem, core);
  if (workspace_bytes < l.total) return TRI_ATTN_ERROR_INSUFFICIENT_WORKSPACE;
  {
    const size_t P = (size_t)problem->B * problem->N * problem->N, E = P * CH * 2;
    const size_t nb = (size_t)problem->B * problem->H * problem->N * problem->N, H = problem->H;
    const Span ins[] = {span(z, E), span(mask, mask ? P : 0), span(dy, E), span(params->ln_w, CH * 4),
                        span(params->ln_b, CH * 4), span(params->w_qkvg, CH * 4 * CH * 2),
                        span(params->w_bias, CH * H * 2), span(params->w_out, CH * CH * 2), span(saved->zn, E),
                        span(saved->ln_stats, P * 8), span(saved->q, E), span(saved->k, E), span(saved->v, E),
                        span(saved->g, E), span(saved->bias, nb * 2), span(saved->o, E),
                        span(saved->o_residual, 2 * E), span(saved->lse, (size_t)problem->B * problem->N * H * problem->N * 4)};
    const Span outs[] = {span(dz, E), span(grads->ln_w, CH * 4), span(grads->ln_b, CH * 4),
                         span(grads->w_qkvg, CH * 4 * CH * 4), span(grads->w_bias, CH * H * 4),
                         span(grads->w_out, CH * CH * 4), span(workspace, l.total)};
    if (!outputs_disjoint(outs, ins)) return TRI_ATTN_ERROR_INVALID_VALUE;
  }
  char *ws = (char *)workspace;
  ModArgs a = base_args(problem);
  a.z = (const uint16_t *)z;
  a.ln_w = params->ln_w;
  a.ln_b = params->ln_b;
  a.w_qkvg = (const uint16_t *)params->w_qkvg;
  a.w_bias = (const uint16_t *)params->w_bias;
  a.w_out = (const uint16_t *)params->w_out;
  a.zn = (uint16_t *)saved->zn;
  a.stats = saved->ln_stats;
  a.g = (uint16_t *)saved->g;
  a.o = (uint16_t *)saved->o;
  a.dy = (const uint16_t *)dy;
  a.d_o = (uint16_t *)(ws + l.off_do);
  a.dgp = (uint16_t *)(ws + l.off_dgp);
  a.dq = (const uint16_t *)(ws + l.off_dq);
  a.dk = (const uint16_t *)(ws + l.off_dk);
  a.dv = (const uint16_t *)(ws + l.off_dv);
  a.dbias = (const float *)(ws + l.off_db);
  a.dz = (uint16_t *)dz;
  a.w_part = (float *)(ws + l.off_w);
  a.ln_part = (float *)(ws + l.off_ln);
  a.slices = l.slices;

  hipLaunchKernelGGL(mod_out_bwd_kernel, dim3((unsigned)a.tiles), dim3(NT), 0, stream, a);
  if (hipGetLastError() != hipSuccess) return TRI_ATTN_ERROR_LAUNCH_FAILED;
  tri_attn_problem cpb = cp;
  cpb.flags |= TRI_ATTN_FLAG_DBIAS_FP32;
  st = tri_attn_bwd(&cpb, saved->q, saved->k, saved->v, saved->bias, mask, saved->o, saved->o_residual, saved->lse,
                    a.d_o, ws + l.off_dq, ws + l.off_dk, ws + l.off_dv, ws + l.off_db, ws + l.off_core, l.core_bytes,
                    stream);
  if (st != TRI_ATTN_SUCCESS) return st;
  hipLaunchKernelGGL(mod_in_bwd_kernel, dim3((unsigned)a.tiles), dim3(NT8), 0, stream, a);
  if (hipGetLastError() != hipSuccess) return TRI_ATTN_ERROR_LAUNCH_FAILED;
  hipLaunchKernelGGL(mod_wgrad_kernel, dim3((unsigned)(6 * a.slices)), dim3(NT8), 0, stream, a);
  if (hipGetLastError() != hipSuccess) return TRI_ATTN_ERROR_LAUNCH_FAILED;
  ReduceArgs r;
  r.w_part = a.w_part;
  r.ln_part = a.ln_part;
  r.dw_qkvg = grads->w_qkvg;
  r.dw_bias = grads->w_bias;
  r.dw_out = grads->w_out;
  r.d_ln_w = grads->ln_w;
  r.d_ln_b = grads->ln_b;
  r.H = a.H;
  r.slices = a.slices;
  r.tiles = a.tiles;
  hipLaunchKernelGGL(mod_reduce_w_kernel, dim3((6 * CH * CH + 255) / 256), dim3(256), 0, stream, r);
  if (hipGetLastError() != hipSuccess) return TRI_ATTN_ERROR_LAUNCH_FAILED;
  hipLaunchKernelGGL(ln_reduce1_kernel, dim3(kLnGroups, 1), dim3(256), 0, stream, r.ln_part, r.ln_part, a.w_part,
                     a.tiles, kLnGroups);
  if (hipGetLastError() != hipSuccess) return TRI_ATTN_ERROR_LAUNCH_FAILED;
  hipLaunchKernelGGL(ln_reduce2_kernel, dim3(4), dim3(256), 0, stream, (const float *)a.w_part, kLnGroups, r.d_ln_w,
                     r.d_ln_b, r.d_ln_w, r.d_ln_b);
  return hipGetLastError() == hipSuccess ? TRI_ATTN_SUCCESS : TRI_ATTN_ERROR_LAUNCH_FAILED;
}

}  // extern "C"
