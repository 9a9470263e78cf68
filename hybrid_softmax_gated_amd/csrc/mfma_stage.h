// LDS staging of the per-head 128x128 operands used by the MFMA kernels.
#pragma once

#include "arl2_device.h"

namespace arl2 {

constexpr int kD = 128;
constexpr int W_LD = kD + 8;  // row stride (bf16) of staged 128x128 tiles: 272 B

__device__ __forceinline__ int swap_bits01(int g) {
  return (g & ~3) | ((g & 1) << 1) | ((g & 2) >> 1);
}

// WT[dout][din] = W[din][dout] for one 128x128 bf16 map stored [din][dout]
// (row stride W_LD), so an operand with k = din reads 16 contiguous bytes.
__device__ __forceinline__ void stage_weight_T(const bf16 *__restrict__ W, bf16 *WT, int tid) {
  for (int u = tid; u < 512; u += 256) {
    const int og = u & 15, ig = u >> 4;
    bf16x8 r[4];
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) r[rr] = *(const bf16x8 *)(W + (4 * ig + rr) * kD + 8 * og);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      bf16x4 t;
      t[0] = r[0][e];
      t[1] = r[1][e];
      t[2] = r[2][e];
      t[3] = r[3][e];
      *(bf16x4 *)(WT + (8 * og + e) * W_LD + 4 * ig) = t;
    }
  }
}

// STh[dv][p] = bf16(S[dk][dv]) with dk = 16*(p/16) + swap_bits23(p%16): the
// k order in which accumulator registers line up with operand positions.
// If STl is not null it receives the bf16 residual S - STh (split-bf16).
__device__ __forceinline__ void stage_state_T(const float *__restrict__ S, bf16 *STh, bf16 *STl,
                                              int tid) {
  for (int u = tid; u < 1024; u += 256) {
    const int vgp = u & 31, kg = u >> 5;
    f32x4 r[4];
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) r[rr] = *(const f32x4 *)(S + (4 * kg + rr) * kD + 4 * vgp);
    const int pos = 16 * (kg >> 2) + 4 * swap_bits01(kg & 3);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      bf16x4 th, tl;
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        bf16 hi, lo;
        split_bf16(r[rr][e], hi, lo);
        th[rr] = hi;
        tl[rr] = lo;
      }
      *(bf16x4 *)(STh + (4 * vgp + e) * W_LD + pos) = th;
      if (STl) *(bf16x4 *)(STl + (4 * vgp + e) * W_LD + pos) = tl;
    }
  }
}

}  // namespace arl2
