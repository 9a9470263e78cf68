// A pure matrix-core loop that measures the bf16 MFMA rate the device
// sustains: the reference next to which the attention kernel's fraction of
// the published dense peak is read.
//
// One 512-thread workgroup per compute unit, so every SIMD holds two
// wavefronts; each wavefront runs `iters` rounds of four independent
// 32x32x16 bf16 MFMA accumulation chains on register operands. Nothing but
// the final accumulators touches memory.
#include "arl2_device.h"
#include "arl2_kernels.h"

namespace arl2 {
namespace {

__global__ __launch_bounds__(512, 1) void mfma_peak_kernel(int iters, float *sink) {
  const int lane = threadIdx.x & 63;
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (bf16)(1e-3f * (float)(lane + i));
    b[i] = (bf16)(1e-3f * (float)(lane - i));
  }
  f32x16 c0 = zero16(), c1 = zero16(), c2 = zero16(), c3 = zero16();
  for (int it = 0; it < iters; ++it) {
    c0 = mfma32(a, b, c0);
    c1 = mfma32(a, b, c1);
    c2 = mfma32(a, b, c2);
    c3 = mfma32(a, b, c3);
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) s += (c0[i] + c1[i]) + (c2[i] + c3[i]);
  sink[(int64_t)blockIdx.x * 512 + threadIdx.x] = s;
}

}  // namespace

hipError_t launch_mfma_peak(int blocks, int iters, float *sink, hipStream_t s) {
  hipLaunchKernelGGL(mfma_peak_kernel, dim3((unsigned)blocks), dim3(512), 0, s, iters, sink);
  return hipGetLastError();
}

double mfma_peak_flops(int blocks, int iters) {
  // 8 wavefronts per workgroup, 4 MFMAs per round, 2*32*32*16 flop each.
  return (double)blocks * 8.0 * 4.0 * (double)iters * 32768.0;
}

}  // namespace arl2
