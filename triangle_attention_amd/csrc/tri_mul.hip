// Triangle multiplicative update: the contraction over the third node of every
// triangle, forward and backward, for MI355X (gfx950, CDNA4).
//
// Operation: the second kernel family of the TurboPairFormer pages (biocloudservice
// page, opening paragraph; Lambda post, opening section), whose cubic-cost core is,
// per channel c and batch b, a contraction over the third node k:
//   outgoing: z[i, j] = sum_k a[i, k] bb[j, k]      incoming: z[i, j] = sum_k a[k, i] bb[k, j]
// and, with g = dL/dz,
//   outgoing: da[i, k] = sum_j g[i, j] bb[j, k],  dbb[j, k] = sum_i g[i, j] a[i, k]
//   incoming: da[k, i] = sum_j g[i, j] bb[k, j],  dbb[k, j] = sum_i g[i, j] a[k, i]
// Tensors are channel-major, [B, C, N, N] (one N x N matrix per channel), so each of
// these six products is a dense N x N x N matrix product per (batch, channel): one
// batched GEMM kernel covers them all,
//   out[m, n] = sum_t L(m, t) R(t, n)
// with each operand stored either with its contraction index t contiguous (row
// reads from LDS) or with m / n contiguous (transposed reads, ds_read_b64_tr_b16).
//
// Kernel: workgroup = a 128 x 128 tile of one (batch, channel) output, 4 waves in a
// 2 x 2 arrangement, each wave 64 x 64 = 2 x 2 products of v_mfma_f32_32x32x16_bf16,
// fp32 accumulation over the whole contraction in registers (one fixed order: results
// are bitwise reproducible), bf16 round-to-nearest-even output.  K steps of 32: the
// next step's operand tiles are loaded into registers while the current one's are
// multiplied out of LDS (two LDS buffers, one barrier per step); the output tile leaves
// through LDS as 16-byte row pieces.  Loading two steps ahead (a second register set)
// measured 35 % slower: its registers cut the workgroups resident per CU from four to
// three, and that concurrency hides more of the load latency than the deeper prefetch.  Workgroups of one
// (batch, channel) follow each other on one XCD (the channel's operands, 2 x 1.2 MB at
// N = 768, stay in that XCD's L2).
//
// MFMA layouts (64 lanes, hh = lane / 32):
//   A (32 x 16): lane supplies A[lane % 32][8 hh + e], e = 0..7
//   B (16 x 32): lane supplies B[8 hh + e][lane % 32]
//   C (32 x 32): lane holds C[8 (r / 4) + 4 hh + r % 4][lane % 32], r = 0..15
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tri_mul.h"

namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) unsigned u32x4;
typedef __attribute__((ext_vector_type(4))) short i16x4;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr int TM = 128, TN = 128, TK = 32;  // workgroup tile and contraction step
constexpr int WAVES = 4;

__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ unsigned pack_bf16(float a, float b) {
  return __builtin_bit_cast(unsigned, __builtin_convertvector((f32x2){a, b}, bf16x2));
}

// Offset (elements) of (row, col) in a [rows][32] bf16 LDS tile whose 16-byte chunks
// are permuted by row bits 2 and 3 (XOR row bit 1, which keeps the index arithmetic
// within the register budget of four workgroups per CU).  With 64 four-byte banks,
// rows r and r + 4 share banks unless their chunks differ, so the 16-byte row reads of
// 16 consecutive rows (one chunk each) then touch every bank once; the transposing
// reads (four consecutive rows per 16-lane group) and the 16-byte piece writes (whole
// rows) are conflict-free under any per-row permutation.
__device__ __forceinline__ int toff(int row, int col) {
  const int sw = ((row >> 2) & 3) ^ (row & 2);
  return row * 32 + (((col >> 3) ^ sw) << 3) + (col & 7);
}

constexpr int SUB = 32 * 32;  // elements of a [32][32] sub-tile

// Row operand of a [rows][32] tile holding (mn, t) with t contiguous: lane gets
// tile[row0 + lane % 32][kk + 8 hh + e].
__device__ __forceinline__ bf16x8 row_operand(const uint16_t *tile, int row0, int kk, int lane) {
  return *(const bf16x8 *)(tile + toff(row0 + (lane & 31), kk + 8 * (lane >> 5)));
}

// Transposed operand of a [32 t][32 mn] tile: lane gets tile[kk + 8 hh + e][lane % 32]
// (column lane % 32 of eight consecutive rows).  ds_read_b64_tr_b16 works on 4 x 16
// blocks: in each 16-lane group, lane 4 m + s addresses row m, columns 4 s .. 4 s + 3,
// and lane c of the group receives column c of the four rows.
__device__ __forceinline__ bf16x8 tr_operand(const uint16_t *tile, int kk, int lane) {
  const int g = lane >> 4, w = lane & 15, m = w >> 2, s = w & 3;
  const int row = kk + 8 * (lane >> 5) + m, col = 16 * (g & 1) + 4 * s;
  i16x4 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(tile + toff(row, col)));
  i16x4 y = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(tile + toff(row + 4, col)));
  typedef __attribute__((ext_vector_type(8))) short i16x8;
  return __builtin_bit_cast(bf16x8, (i16x8)__builtin_shufflevector(x, y, 0, 1, 2, 3, 4, 5, 6, 7));
}

// Workgroup index -> tile index such that consecutive tiles share an XCD
// (workgroups are dealt to the 8 XCDs round-robin).
__device__ __forceinline__ int xcd_remap(int L, int G) {
  const int per = G >> 3;
  if (L < (per << 3)) return (L & 7) * per + (L >> 3);
  return L;
}

struct GemmArgs {
  const uint16_t *L, *R;  // operands, [B * C][N][N] each
  uint16_t *out;          // [B * C][N][N]
  int N, batches, tiles;  // tiles per side: ceil(N / 128)
};

// One 128 x 32 operand tile per step, as 16-byte pieces: 512 pieces, two per thread.
//   t contiguous (TR = false): piece p -> row mn = p / 4, t = 8 (p % 4); stored [mn][t]
//     in four [32][32] sub-tiles (mn / 32).
//   mn contiguous (TR = true): stored [t][mn] in four [32 t][32 mn] sub-tiles (mn / 32);
//     each 16 consecutive pieces cover rows t .. t + 3 of one sub-tile (four 64-byte row
//     segments: piece p -> sub-tile (p / 16) % 4, t = 4 (p / 64) + (p % 16) / 4,
//     mn = 32 sub + 8 (p % 4)), so that a 16-lane LDS write covers every bank once.
// Rows past N (a ragged last tile) load zeros.
template <bool TR>
struct TileIO {
  __device__ static void load(const uint16_t *mat, int N, int mn0, int t0, int tid, u32x4 *w) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int p = tid + 256 * i;
      int r, c;
      if (TR) {
        r = t0 + 4 * (p >> 6) + ((p & 15) >> 2);
        c = mn0 + 32 * ((p >> 4) & 3) + 8 * (p & 3);
      } else {
        r = mn0 + (p >> 2);
        c = t0 + 8 * (p & 3);
      }
      const bool in = TR ? (c < N) : (r < N);
      const long long off = (long long)min(r, N - 1) * N + min(c, N - 8);
      const u32x4 v = *(const u32x4 *)(mat + off);
      w[i] = in ? v : (u32x4){0u, 0u, 0u, 0u};
    }
  }
  __device__ static void store(uint16_t *lds, int tid, const u32x4 *w) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int p = tid + 256 * i;
      int sub, row, col;
      if (TR) {
        sub = (p >> 4) & 3;
        row = 4 * (p >> 6) + ((p & 15) >> 2);
        col = 8 * (p & 3);
      } else {
        const int mn = p >> 2;
        sub = mn >> 5;
        row = mn & 31;
        col = 8 * (p & 3);
      }
      *(u32x4 *)(lds + sub * SUB + toff(row, col)) = w[i];
    }
  }
  // operand for the 32 rows / columns mn32 .. mn32 + 31 of the tile, t = kk .. kk + 15
  __device__ static bf16x8 operand(const uint16_t *lds, int mn32, int kk, int lane) {
    const uint16_t *sub = lds + (mn32 >> 5) * SUB;
    return TR ? tr_operand(sub, kk, lane) : row_operand(sub, 0, kk, lane);
  }
};

// out[m, n] = sum_t L(m, t) R(t, n) per (batch, channel):
//   LT = false: L stored [m][t];  LT = true: L stored [t][m]
//   RT = false: R stored [n][t];  RT = true: R stored [t][n]
template <bool LT, bool RT>
__global__ __launch_bounds__(WAVES * 64, 2) void tri_mul_gemm(GemmArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * (TM + TN) * TK];
  uint16_t (*sL)[TM * TK] = (uint16_t (*)[TM * TK])smem;
  uint16_t (*sR)[TN * TK] = (uint16_t (*)[TN * TK])(smem + 2 * TM * TK);
  const int N = a.N;
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hh = lane >> 5, ll = lane & 31;
  int t = xcd_remap(blockIdx.x, gridDim.x);
  const int per = a.tiles * a.tiles;
  const int bc = t / per;
  t -= bc * per;
  const int m0 = (t / a.tiles) * TM, n0 = (t % a.tiles) * TN;
  const long long mat = (long long)bc * N * N;
  const uint16_t *L = a.L + mat, *R = a.R + mat;
  const int wm = (wave >> 1) * 64, wn = (wave & 1) * 64;  // the wave's 64 x 64 part

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = (f32x16){};

  u32x4 wl[2], wr[2];
  TileIO<LT>::load(L, N, m0, 0, tid, wl);
  TileIO<RT>::load(R, N, n0, 0, tid, wr);
  TileIO<LT>::store(sL[0], tid, wl);
  TileIO<RT>::store(sR[0], tid, wr);
  __syncthreads();
  const int nk = N / TK;
  for (int ks = 0; ks < nk; ++ks) {
    const int cur = ks & 1;
    const bool more = ks + 1 < nk;
    if (more) {  // the next step's tiles into registers
      TileIO<LT>::load(L, N, m0, (ks + 1) * TK, tid, wl);
      TileIO<RT>::load(R, N, n0, (ks + 1) * TK, tid, wr);
    }
#pragma unroll
    for (int kk = 0; kk < TK; kk += 16) {
      bf16x8 la[2], rb[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        la[i] = TileIO<LT>::operand(sL[cur], wm + 32 * i, kk, lane);
        rb[i] = TileIO<RT>::operand(sR[cur], wn + 32 * i, kk, lane);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = mfma(la[i], rb[j], acc[i][j]);
    }
    if (more) {
      TileIO<LT>::store(sL[cur ^ 1], tid, wl);
      TileIO<RT>::store(sR[cur ^ 1], tid, wr);
    }
    __syncthreads();
  }

  // bf16 output through LDS: lane holds rows 8 (r / 4) + 4 hh + r % 4 of column ll of
  // each product; the staged [128][128] tile leaves as 16-byte row pieces
  uint16_t *so = smem;  // [TM][TN], 16-byte chunks permuted per row like the step tiles
  auto ooff = [](int row, int col) { return row * TN + (((col >> 3) ^ (row & 15)) << 3) + (col & 7); };
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = wm + 32 * i + 8 * (r >> 2) + 4 * hh + (r & 3), n = wn + 32 * j + ll;
        so[ooff(m, n)] = (uint16_t)(pack_bf16(acc[i][j][r], 0.f) & 0xffffu);
      }
  __syncthreads();
  uint16_t *out = a.out + mat;
#pragma unroll
  for (int i = 0; i < (TM * TN / 8) / (WAVES * 64); ++i) {
    const int pc = tid + WAVES * 64 * i, row = pc / (TN / 8), c = (pc % (TN / 8)) * 8;
    const int m = m0 + row, n = n0 + c;
    if (m < N && n < N) *(u32x4 *)(out + (long long)m * N + n) = *(const u32x4 *)(so + ooff(row, c));
  }
}

// ------------------------------------------------------------------------------------
// Host side
// ------------------------------------------------------------------------------------
constexpr int64_t kMaxN = 1024;
constexpr int64_t kMaxBC = 1 << 16;

bool aligned16(const void *p) { return p && ((uintptr_t)p & 15u) == 0; }

struct Range {
  uintptr_t lo, hi;
};
Range span(const void *p, size_t bytes) { return {(uintptr_t)p, (uintptr_t)p + bytes}; }
bool overlap(Range x, Range y) { return x.lo < y.hi && y.lo < x.hi; }

tri_attn_status check(const tri_mul_problem *p) {
  if (!p) return TRI_ATTN_ERROR_INVALID_VALUE;
  if (p->abi_version != TRI_MUL_ABI_VERSION) return TRI_ATTN_ERROR_ABI_MISMATCH;
  if (p->B < 1 || p->N < 1 || p->C < 1) return TRI_ATTN_ERROR_INVALID_VALUE;
  if (p->flags & ~TRI_MUL_FLAG_INCOMING) return TRI_ATTN_ERROR_NOT_SUPPORTED;
  if (p->N % 32 != 0 || p->N > kMaxN || p->B * p->C > kMaxBC) return TRI_ATTN_ERROR_NOT_SUPPORTED;
  return TRI_ATTN_SUCCESS;
}

template <bool LT, bool RT>
hipError_t launch(const void *L, const void *R, void *out, const tri_mul_problem &p, hipStream_t stream) {
  GemmArgs a;
  a.L = (const uint16_t *)L;
  a.R = (const uint16_t *)R;
  a.out = (uint16_t *)out;
  a.N = (int)p.N;
  a.batches = (int)(p.B * p.C);
  a.tiles = (int)((p.N + TM - 1) / TM);
  const unsigned grid = (unsigned)(a.batches * a.tiles * a.tiles);
  auto kern = tri_mul_gemm<LT, RT>;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(WAVES * 64), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

extern "C" {

int tri_mul_abi_version(void) { return TRI_MUL_ABI_VERSION; }

tri_attn_status tri_mul_fwd(const tri_mul_problem *problem, const void *a, const void *b, void *z,
                            hipStream_t stream) {
  const tri_attn_status st = check(problem);
  if (st != TRI_ATTN_SUCCESS) return st;
  const tri_mul_problem &p = *problem;
  if (!aligned16(a) || !aligned16(b) || !aligned16(z)) return TRI_ATTN_ERROR_INVALID_VALUE;
  const size_t bytes = (size_t)p.B * p.C * p.N * p.N * 2;
  if (overlap(span(z, bytes), span(a, bytes)) || overlap(span(z, bytes), span(b, bytes)))
    return TRI_ATTN_ERROR_INVALID_VALUE;
  // outgoing: z[i, j] = sum_k a[i, k] b[j, k]  (L = a [m][t], R = b [n][t])
  // incoming: z[i, j] = sum_k a[k, i] b[k, j]  (L = a [t][m], R = b [t][n])
  const bool in = (p.flags & TRI_MUL_FLAG_INCOMING) != 0;
  const hipError_t e = in ? launch<true, true>(a, b, z, p, stream) : launch<false, false>(a, b, z, p, stream);
  return e == hipSuccess ? TRI_ATTN_SUCCESS : TRI_ATTN_ERROR_LAUNCH_FAILED;
}

tri_attn_status tri_mul_bwd(const tri_mul_problem *problem, const void *a, const void *b, const void *dz,
                            void *da, void *db, hipStream_t stream) {
  const tri_attn_status st = check(problem);
  if (st != TRI_ATTN_SUCCESS) return st;
  const tri_mul_problem &p = *problem;
  if (!aligned16(a) || !aligned16(b) || !aligned16(dz) || !aligned16(da) || !aligned16(db))
    return TRI_ATTN_ERROR_INVALID_VALUE;
  const size_t bytes = (size_t)p.B * p.C * p.N * p.N * 2;
  const Range ins[] = {span(a, bytes), span(b, bytes), span(dz, bytes)};
  const Range outs[] = {span(da, bytes), span(db, bytes)};
  for (const Range &x : outs)
    for (const Range &y : ins)
      if (overlap(x, y)) return TRI_ATTN_ERROR_INVALID_VALUE;
  if (overlap(outs[0], outs[1])) return TRI_ATTN_ERROR_INVALID_VALUE;
  const bool in = (p.flags & TRI_MUL_FLAG_INCOMING) != 0;
  hipError_t e;
  if (!in) {
    // da[i, k] = sum_j g[i, j] b[j, k]   (L = g [m][t], R = b [t][n])
    e = launch<false, true>(dz, b, da, p, stream);
    // db[j, k] = sum_i g[i, j] a[i, k]   (L = g [t][m], R = a [t][n])
    if (e == hipSuccess) e = launch<true, true>(dz, a, db, p, stream);
  } else {
    // da[k, i] = sum_j b[k, j] g[i, j]   (L = b [m][t], R = g [n][t])
    e = launch<false, false>(b, dz, da, p, stream);
    // db[k, j] = sum_i a[k, i] g[i, j]   (L = a [m][t], R = g [t][n])
    if (e == hipSuccess) e = launch<false, true>(a, dz, db, p, stream);
  }
  return e == hipSuccess ? TRI_ATTN_SUCCESS : TRI_ATTN_ERROR_LAUNCH_FAILED;
}

}  // extern "C"
