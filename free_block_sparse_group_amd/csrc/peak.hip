// Matrix-core rate probe (measurement only, not part of the method): the
// sustained bf16 dense MFMA rate of the chip at the clock it runs under load,
// reported beside the 2.5 PFLOP/s specification.
#include "common.hpp"
#include "kernels.hpp"

namespace spr {

// Each wave keeps four independent 32x32 accumulators and issues four
// v_mfma_f32_32x32x16_bf16 per round on register operands (no memory
// traffic in the loop); the accumulators' sum is written once per thread.
__global__ __launch_bounds__(256) void k_mfma_rate(int iters, float* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (bf16_t)(1.0f + 0.001f * (float)((lane + i) & 7));
    b[i] = (bf16_t)(0.5f - 0.001f * (float)((lane * 3 + i) & 7));
  }
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int it = 0; it < iters; ++it) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, a, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, a, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, b, c3, 0, 0, 0);
  }
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) s += (c0[i] + c1[i]) + (c2[i] + c3[i]);
  sink[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

hipError_t launch_mfma_rate(int blocks, int iters, float* sink, hipStream_t st) {
  hipLaunchKernelGGL(k_mfma_rate, dim3(blocks), dim3(256), 0, st, iters, sink);
  return hipGetLastError();
}

}  // namespace spr
