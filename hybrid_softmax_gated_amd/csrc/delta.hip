// Gated delta state update of the inter-frame branch (bf16 io, d = 128).
//
// Method: "Technical Summary: Attend Locally, Remember Linearly (ARL2)",
// section 2.1 (state update) and section 2.2 (the state is written once per
// frame, after the clean pass, from the pre-update state):
//   K' = L2norm(k W_k), V' = v W_v, R = V' - K' S_{N-1},
//   S_N = alpha S_{N-1} + K'^T diag(beta) R.
//
// Work split: one workgroup per chunk of 128 tokens of one (stream, head)
// computes that chunk's contribution dS_c = K'_c^T diag(beta_c) R_c into the
// workspace; a second kernel applies S = alpha S + sum_c dS_c in a fixed
// chunk order (deterministic, no atomics). Every workgroup of the first
// kernel reads the same pre-update S, so the in-place write is safe.
//
// Precision: the feature maps use bf16 operands (the inputs are bf16) with
// fp32 accumulation, which is exact per product. The two products that
// involve the fp32 state or the fp32 K' — K'S and K'^T (beta R) — use the
// split-bf16 scheme (x = hi + lo, three MFMAs hi*hi + hi*lo + lo*hi; Henry,
// Tang and Heinecke, ARITH 2019), about 2^-16 relative per product, because
// plain bf16 operands lose about 2^-9 per frame on the state.
//
// Per wavefront (32 tokens), phase 1:
//   (1) (k W_k)^T with lanes = tokens -> in-register L2 norms -> K'
//   (2) V' = v W_v with lanes = d_v, registers = tokens
//   (3) K'S with the same layout as V', K' fed from (1)'s accumulators
//   (4) beta (V' - K'S)
//   (5) K' again with lanes = d_k, registers = tokens (the layout the
//       contraction over tokens needs), scaled by (1)'s norms
// Phase 2: (4) and (5) of all four wavefronts go to LDS in register order;
// wavefront w then forms rows 32w .. 32w+31 of dS_c over the 128 tokens.
#include "arl2_device.h"
#include "arl2_kernels.h"
#include "mfma_stage.h"

#include <math.h>

namespace arl2 {
namespace {

constexpr int D = 128;
constexpr int TILE = D * W_LD;              // bf16 elements of one staged 128x128 tile
constexpr int SPILL = 4 * 4 * 64 * 16;      // bf16 elements: [wave][block][lane][16 regs]

struct DeltaKParams {
  const bf16 *k, *v, *Wk, *Wv;
  const float *S, *beta;
  int H, L, nchunk;
  float *ws_dS;
};

__global__ __launch_bounds__(256) void delta_partial_kernel(DeltaKParams p) {
  // Phase 1: W_k^T, W_v^T, S^T (hi, lo). Phase 2 reuses the same bytes.
  __shared__ __attribute__((aligned(16))) bf16 lds[4 * TILE];
  __shared__ float betas[kDeltaChunk];
  __shared__ float invn[kDeltaChunk];
  bf16 *WkT = lds, *WvT = lds + TILE, *STh = lds + 2 * TILE, *STl = lds + 3 * TILE;
  bf16 *Kh = lds, *Kl = lds + SPILL, *Rh = lds + 2 * SPILL, *Rl = lds + 3 * SPILL;

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, hl = lane >> 5, l32 = lane & 31;
  const int chunk = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int64_t tok = (int64_t)p.H * D;
  const int tbase = chunk * kDeltaChunk;

  stage_weight_T(p.Wk + (int64_t)h * D * D, WkT, tid);
  stage_weight_T(p.Wv + (int64_t)h * D * D, WvT, tid);
  stage_state_T(p.S + ((int64_t)b * p.H + h) * D * D, STh, STl, tid);
  if (tid < kDeltaChunk) {
    const int t = tbase + tid;
    betas[tid] = t < p.L ? p.beta[((int64_t)b * p.L + t) * p.H + h] : 0.f;
  }
  __syncthreads();

  // This wavefront's 32 tokens: lane l holds token l%32, features 16c + 8*(l/32) .. +7.
  const int trow = tbase + 32 * wave + l32;
  bf16x8 kop[8], vop[8];
  if (trow < p.L) {
    const int64_t off = ((int64_t)b * p.L * p.H + h) * D + trow * tok + 8 * hl;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      kop[c] = *(const bf16x8 *)(p.k + off + 16 * c);
      vop[c] = *(const bf16x8 *)(p.v + off + 16 * c);
    }
  } else {
#pragma unroll
    for (int c = 0; c < 8; ++c) kop[c] = vop[c] = zero_bf16x8();
  }

  // (1) (k W_k)^T: lane = token, registers = d_k.
  f32x16 kt[4];
#pragma unroll
  for (int bb = 0; bb < 4; ++bb) {
    kt[bb] = zero16();
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const bf16x8 a = *(const bf16x8 *)(WkT + (32 * bb + l32) * W_LD + 16 * c + 8 * hl);
      kt[bb] = mfma32(a, kop[c], kt[bb]);
    }
  }
  float ss = 0.f;
#pragma unroll
  for (int bb = 0; bb < 4; ++bb)
#pragma unroll
    for (int i = 0; i < 16; ++i) ss = fmaf(kt[bb][i], kt[bb][i], ss);
  ss += swap_halves(ss);
  const float inv = 1.f / fmaxf(sqrtf(ss), kL2Eps);
  if (hl == 0) invn[32 * wave + l32] = inv;

  // (2) V' = v W_v: lane = d_v, registers = tokens.
  f32x16 r[4];
#pragma unroll
  for (int bb = 0; bb < 4; ++bb) {
    r[bb] = zero16();
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const bf16x8 bw = *(const bf16x8 *)(WvT + (32 * bb + l32) * W_LD + 16 * c + 8 * hl);
      r[bb] = mfma32(vop[c], bw, r[bb]);
    }
  }

  // (3) K'S, split-bf16 on both operands: K' straight from (1)'s registers.
  f32x16 ks[4];
#pragma unroll
  for (int bb = 0; bb < 4; ++bb) ks[bb] = zero16();
#pragma unroll
  for (int g = 0; g < 8; ++g) {
    bf16x8 ah, al;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      bf16 hi, lo;
      split_bf16(kt[g >> 1][8 * (g & 1) + j] * inv, hi, lo);
      ah[j] = hi;
      al[j] = lo;
    }
#pragma unroll
    for (int bb = 0; bb < 4; ++bb) {
      const int off = (32 * bb + l32) * W_LD + 16 * g + 8 * hl;
      const bf16x8 sh = *(const bf16x8 *)(STh + off);
      const bf16x8 sl = *(const bf16x8 *)(STl + off);
      ks[bb] = mfma32(ah, sh, ks[bb]);
      ks[bb] = mfma32(ah, sl, ks[bb]);
      ks[bb] = mfma32(al, sh, ks[bb]);
    }
  }

  __syncthreads();  // invn complete

  // (4) beta (V' - K'S), rows = tokens.
#pragma unroll
  for (int bb = 0; bb < 4; ++bb)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int t = 32 * wave + 8 * (i >> 2) + 4 * hl + (i & 3);
      r[bb][i] = (r[bb][i] - ks[bb][i]) * betas[t];
    }

  // (5) K' with lane = d_k, registers = tokens.
  f32x16 kr[4];
#pragma unroll
  for (int bb = 0; bb < 4; ++bb) {
    kr[bb] = zero16();
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const bf16x8 bw = *(const bf16x8 *)(WkT + (32 * bb + l32) * W_LD + 16 * c + 8 * hl);
      kr[bb] = mfma32(kop[c], bw, kr[bb]);
    }
  }
  float tinv[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) tinv[i] = invn[32 * wave + 8 * (i >> 2) + 4 * hl + (i & 3)];

  __syncthreads();  // all reads of the staged weights and state are done

  // Spill (4) and (5) in register order: [wave][block][lane][16].
#pragma unroll
  for (int bb = 0; bb < 4; ++bb) {
    bf16x8 kh0, kh1, kl0, kl1, rh0, rh1, rl0, rl1;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      bf16 hi, lo;
      split_bf16(kr[bb][j] * tinv[j], hi, lo);
      kh0[j] = hi;
      kl0[j] = lo;
      split_bf16(kr[bb][8 + j] * tinv[8 + j], hi, lo);
      kh1[j] = hi;
      kl1[j] = lo;
      split_bf16(r[bb][j], hi, lo);
      rh0[j] = hi;
      rl0[j] = lo;
      split_bf16(r[bb][8 + j], hi, lo);
      rh1[j] = hi;
      rl1[j] = lo;
    }
    const int off = ((wave * 4 + bb) * 64 + lane) * 16;
    *(bf16x8 *)(Kh + off) = kh0;
    *(bf16x8 *)(Kh + off + 8) = kh1;
    *(bf16x8 *)(Kl + off) = kl0;
    *(bf16x8 *)(Kl + off + 8) = kl1;
    *(bf16x8 *)(Rh + off) = rh0;
    *(bf16x8 *)(Rh + off + 8) = rh1;
    *(bf16x8 *)(Rl + off) = rl0;
    *(bf16x8 *)(Rl + off + 8) = rl1;
  }
  __syncthreads();

  // Phase 2: rows d_k in [32*wave, 32*wave + 32) of dS_c, all d_v.
  f32x16 ds[4];
#pragma unroll
  for (int bb = 0; bb < 4; ++bb) ds[bb] = zero16();
  for (int pw = 0; pw < 4; ++pw) {
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      const int aoff = ((pw * 4 + wave) * 64 + lane) * 16 + 8 * st;
      const bf16x8 ah = *(const bf16x8 *)(Kh + aoff);
      const bf16x8 al = *(const bf16x8 *)(Kl + aoff);
#pragma unroll
      for (int bb = 0; bb < 4; ++bb) {
        const int boff = ((pw * 4 + bb) * 64 + lane) * 16 + 8 * st;
        const bf16x8 bh = *(const bf16x8 *)(Rh + boff);
        const bf16x8 bl = *(const bf16x8 *)(Rl + boff);
        ds[bb] = mfma32(ah, bh, ds[bb]);
        ds[bb] = mfma32(ah, bl, ds[bb]);
        ds[bb] = mfma32(al, bh, ds[bb]);
      }
    }
  }

  float *wd = p.ws_dS + (((int64_t)b * p.H + h) * p.nchunk + chunk) * D * D;
#pragma unroll
  for (int bb = 0; bb < 4; ++bb)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int dk = 32 * wave + 8 * (i >> 2) + 4 * hl + (i & 3);
      wd[dk * D + 32 * bb + l32] = ds[bb][i];
    }
}

__global__ __launch_bounds__(256) void delta_apply_kernel(float *S, const float *alpha,
                                                          const float *ws, int dd, int nchunk) {
  const int e = blockIdx.x * 256 + threadIdx.x;
  const int bh = blockIdx.y;
  if (e >= dd) return;
  const float *w = ws + (int64_t)bh * nchunk * dd + e;
  float acc = 0.f;
  for (int c = 0; c < nchunk; ++c) acc += w[(int64_t)c * dd];
  float *sp = S + (int64_t)bh * dd + e;
  *sp = fmaf(alpha[bh], *sp, acc);
}

__global__ __launch_bounds__(256) void fill_state_kernel(float *dst, const float *src, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) dst[i] = src ? src[i] : 0.f;
}

}  // namespace

hipError_t launch_delta_partial_bf16(const DeltaArgs &a, hipStream_t s) {
  DeltaKParams p;
  p.k = (const bf16 *)a.k;
  p.v = (const bf16 *)a.v;
  p.Wk = (const bf16 *)a.Wk;
  p.Wv = (const bf16 *)a.Wv;
  p.S = a.S;
  p.beta = a.beta;
  p.H = a.H;
  p.L = a.L;
  p.nchunk = a.nchunk;
  p.ws_dS = a.ws_dS;
  dim3 grid((unsigned)a.nchunk, (unsigned)a.H, (unsigned)a.B);
  hipLaunchKernelGGL(delta_partial_kernel, grid, dim3(256), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_delta_apply(float *S, const float *alpha, const float *ws_dS, int B, int H,
                              int d, int nchunk, hipStream_t s) {
  const int dd = d * d;
  dim3 grid((unsigned)((dd + 255) / 256), (unsigned)(B * H));
  hipLaunchKernelGGL(delta_apply_kernel, grid, dim3(256), 0, s, S, alpha, ws_dS, dd, nchunk);
  return hipGetLastError();
}

hipError_t launch_fill_state(float *dst, const float *src, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  dim3 grid((unsigned)((n + 255) / 256));
  hipLaunchKernelGGL(fill_state_kernel, grid, dim3(256), 0, s, dst, src, n);
  return hipGetLastError();
}

}  // namespace arl2
