// Matrix-core throughput probe (measurement support for the roofline).
//
// Every wave issues `iters` rounds of four independent
// v_mfma_f32_32x32x16_bf16 chains (operands held in registers, no memory
// traffic in the loop), on 4 workgroups of 8 waves per compute unit.  The rate
// this reaches under the card's own clock management is the practical bf16
// ceiling that the attention kernels are compared with, next to the public
// dense figure of 256 CU x 2.4 GHz x 4096 flop/clk.
#include "kcommon.h"
#include "kernels.h"

namespace ra {

__global__ __launch_bounds__(512) void mfma_rate_kernel(int iters, float* sink) {
  const int lane = threadIdx.x & 63;
  // small nonzero bf16 operands that differ per lane (keeps the datapath toggling)
  float xa[8], xb[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    xa[e] = 0.001f * (float)((lane * 7 + e * 3) % 17 - 8);
    xb[e] = 0.001f * (float)((lane * 5 + e * 11) % 13 - 6);
  }
  const Frag<bf16_storage> a = frag_from_f32<bf16_storage>(xa);
  const Frag<bf16_storage> b = frag_from_f32<bf16_storage>(xb);
  f32x16_t c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int i = 0; i < iters; ++i) {
    mma(c0, a, b);
    mma(c1, b, a);
    mma(c2, a, a);
    mma(c3, b, b);
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) s += c0[i] + c1[i] + c2[i] + c3[i];
  if (threadIdx.x == 0) sink[blockIdx.x] = s;
}

hipError_t launch_mfma_rate(int iters, float* sink, int blocks, hipStream_t st) {
  hipLaunchKernelGGL(mfma_rate_kernel, dim3(blocks), dim3(512), 0, st, iters, sink);
  return hipGetLastError();
}

}  // namespace ra
