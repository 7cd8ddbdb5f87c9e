// Sustained rate of the bf16 matrix cores of this device, measured by bench.py next
// to the published MI355X peak.  It is a measurement aid, not part of the
// triangle-attention library: every wave issues v_mfma_f32_32x32x16_bf16 back to
// back on four independent accumulators, so the matrix pipe never waits for a
// result, and the only memory access is one store per thread at the end.
#include <hip/hip_runtime.h>

namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) unsigned u32x4;

__global__ __launch_bounds__(256) void mfma_probe_kernel(float *out, int iters) {
  const unsigned t = threadIdx.x;
  // operands are bf16 1.0 and 1 + k/128 (k = t % 8), built from the thread index so
  // that they are not compile-time constants; 16-term sums of such products stay far
  // inside the fp32 range for any iteration count used here
  const unsigned one = 0x3f80u, var = 0x3f80u | (t & 7u);
  const u32x4 wa = {one | (one << 16), one | (var << 16), one | (one << 16), var | (one << 16)};
  const u32x4 wb = {var | (one << 16), one | (one << 16), one | (var << 16), one | (one << 16)};
  const bf16x8 a = __builtin_bit_cast(bf16x8, wa), b = __builtin_bit_cast(bf16x8, wb);
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int i = 0; i < iters; ++i) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) s += c0[i] + c1[i] + c2[i] + c3[i];
  out[(long long)blockIdx.x * blockDim.x + t] = s;
}

}  // namespace

// Launches `blocks` workgroups of 256 threads (four waves), each wave running
// `iters` rounds of four 32x32x16 bf16 products (4 * 32768 flop per round), on
// `stream`.  out must hold blocks * 256 floats of device memory.  Returns 0, 1 for
// an invalid argument (nothing launched) or 4 if the launch failed.
extern "C" int mfma_probe_launch(float *out, int blocks, int iters, hipStream_t stream) {
  if (!out || blocks < 1 || iters < 1) return 1;
  hipLaunchKernelGGL(mfma_probe_kernel, dim3(blocks), dim3(256), 0, stream, out, iters);
  return hipGetLastError() == hipSuccess ? 0 : 4;
}
