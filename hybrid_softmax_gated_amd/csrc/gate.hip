// Gate projections of one frame: the delta rule's learning rate beta (one
// value per token and head) and forget gate alpha (one value per head and
// frame) computed from the tokens that enter the layer.
//
// "Technical Summary: Attend Locally, Remember Linearly (ARL2)", section 2.1:
// both gates are learned per-token projections; section 4 (ablations): the
// forget gate is headwise. One forget gate per frame needs the per-token
// values pooled; this library pools the logits by their mean over the
// frame's tokens:
//   beta[b][t][h] = sigmoid(x[b][t] . Wb[h])
//   alpha[b][h]   = sigmoid(mean_t x[b][t] . Wa[h])
//
// Both are one skinny product Z = x [Wa; Wb]^T (B*L rows, 2H columns, D deep)
// followed by elementwise work, so:
//   1. gate_logits: Z on the matrix cores. A workgroup takes 16 tokens x 32
//      gate columns over all of D; its eight wavefronts each take an eighth
//      of D, staging the rows they need through LDS in whole cache lines,
//      and their accumulators are summed in LDS in wave order. Beta is
//      finished in place; the alpha logits of the 16 tokens are summed (in
//      token order) into one partial per head in the workspace.
//   2. gate_alpha: per stream and head, one wavefront sums the partials in a
//      fixed order, divides by L and writes alpha.
// x is read once; the weights (2H x D) stay in L2. No atomics, so the
// results are bitwise reproducible.
#include "arl2_device.h"
#include "arl2_kernels.h"

namespace arl2 {
namespace {

constexpr int kGTok = 16;    // tokens per workgroup
constexpr int kGCols = 32;   // gate columns per workgroup (two 16-column MFMA tiles)
constexpr int kGGroup = 64;  // elements of D per group (two MFMA steps of 32)
constexpr int kGWaves = 8;   // wavefronts per workgroup, each with 1/8 of D
constexpr int kGBatch = 3;   // groups staged per wavefront at a time
constexpr int kGRows = kGTok + kGCols;                // staged rows: 16 of x, 32 of weights
constexpr int kGStage = kGBatch * kGRows * 128;       // bytes of staging per wavefront

__device__ __forceinline__ float sigmoid(float z) { return 1.f / (1.f + expf(-z)); }

struct GateLogitParams {
  const bf16 *x;        // [B][L][D]
  const bf16 *Wa, *Wb;  // [H][D]
  int B, L, D, H;
  int ntt, nnt;         // token tiles, column tiles
  float *beta;          // [B][L][H]
  float *za;            // [B][ntt][H]: alpha logits summed over a token tile
};

// Each wavefront walks its share of D in groups of 64 elements (128 bytes
// of every row). A group's 48 rows (16 token rows of x, 32 weight rows) are
// copied to the wavefront's LDS staging area with whole 128-byte lines per
// 8 lanes; 16-byte chunk c of staged row R sits at position c ^ (R & 7) so
// that the operand reads below (16 rows, same chunk) spread over the banks.
// MFMA step s of a group takes, on lane quarter q, chunk 2q + s of each row:
// the order in which D is walked does not change Z = sum_k x_k w_k other
// than by rounding, and both operands walk it the same way.
__global__ __launch_bounds__(kGWaves * 64) void gate_logits_mfma(GateLogitParams p) {
  __shared__ __attribute__((aligned(16))) char stage[kGWaves][kGStage];
  __shared__ float zt[kGTok][kGCols + 1];
  int bid = blockIdx.x;
  const int tt = bid % p.ntt;
  bid /= p.ntt;
  const int nt = bid % p.nnt;
  const int b = bid / p.nnt;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;

  // Source row of each staged row this lane copies: lane i copies chunk
  // (i % 8) ^ (R & 7) of row R = 8n + i / 8 for n = 0..5. Rows past the
  // frame's end or past the 2H gate columns read a valid row instead; what
  // they produce is never stored.
  const bf16 *src[kGRows / 8];
#pragma unroll
  for (int n = 0; n < kGRows / 8; ++n) {
    const int R = 8 * n + (lane >> 3);
    const int chunk = (lane & 7) ^ (R & 7);
    const bf16 *row;
    if (R < kGTok) {
      const int t = tt * kGTok + R;
      row = p.x + ((int64_t)b * p.L + (t < p.L ? t : 0)) * p.D;
    } else {
      const int cg = nt * kGCols + (R - kGTok);
      row = cg < p.H ? p.Wa + (int64_t)cg * p.D
                     : cg < 2 * p.H ? p.Wb + (int64_t)(cg - p.H) * p.D : p.Wa;
    }
    src[n] = row + 8 * chunk;
  }
  char *my = stage[wave];
  const int r = lane & 15, q = lane >> 4;
  const int G = p.D / kGGroup;
  const int g0 = wave * G / kGWaves, g1 = (wave + 1) * G / kGWaves;

  f32x4 acc[2] = {zero4(), zero4()};
  for (int gb = g0; gb < g1; gb += kGBatch) {
    const int nb = g1 - gb < kGBatch ? g1 - gb : kGBatch;
    for (int j = 0; j < nb; ++j)
#pragma unroll
      for (int n = 0; n < kGRows / 8; ++n)
        global_to_lds16(src[n] + (gb + j) * kGGroup, my + (j * kGRows + 8 * n) * 128);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    for (int j = 0; j < nb; ++j) {
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        const int c = (2 * q + st) ^ (r & 7);
        const bf16x8 a = *(const bf16x8 *)(my + ((j * kGRows + r) * 8 + c) * 16);
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) {
          const bf16x8 w =
              *(const bf16x8 *)(my + ((j * kGRows + kGTok + 16 * ct + r) * 8 + c) * 16);
          acc[ct] = mfma16(a, w, acc[ct]);
        }
      }
    }
    // The next batch overwrites the staging area; its reads above have all
    // been consumed by the MFMAs.
  }
  __syncthreads();
  // Staging is free now: reuse it for the eight wavefronts' accumulators.
  float(*red)[64][9] = reinterpret_cast<float(*)[64][9]>(&stage[0][0]);
#pragma unroll
  for (int ct = 0; ct < 2; ++ct)
#pragma unroll
    for (int i = 0; i < 4; ++i) red[wave][lane][4 * ct + i] = acc[ct][i];
  __syncthreads();

  // Thread e: row e / 32, column e % 32 of the 16 x 32 tile. Accumulator
  // register i of lane l in column tile ct holds row 4(l/16) + i, column
  // 16 ct + l%16.
  {
    const int e = threadIdx.x;
    const int row = e >> 5, c = e & 31;
    const int ct = c >> 4;
    const int l = 16 * (row >> 2) + (c & 15), i = 4 * ct + (row & 3);
    float z = red[0][l][i];
#pragma unroll
    for (int w = 1; w < kGWaves; ++w) z += red[w][l][i];
    zt[row][c] = z;
    const int t = tt * kGTok + row, cg = nt * kGCols + c;
    if (t < p.L && cg >= p.H && cg < 2 * p.H)
      p.beta[((int64_t)b * p.L + t) * p.H + (cg - p.H)] = sigmoid(z);
  }
  __syncthreads();
  // Alpha columns: the tile's tokens summed in token order.
  const int cg = nt * kGCols + (int)threadIdx.x;
  if (threadIdx.x < kGCols && cg < p.H) {
    const int nrow = p.L - tt * kGTok < kGTok ? p.L - tt * kGTok : kGTok;
    float sacc = 0.f;
    for (int row = 0; row < nrow; ++row) sacc += zt[row][threadIdx.x];
    p.za[((int64_t)b * p.ntt + tt) * p.H + cg] = sacc;
  }
}

// Any dtype, any D: one thread per (token, gate column), fp32 FMA chain.
// Beta is finished in place; the alpha logits go to the workspace one per
// token (so a "tile" here is one token).
template <typename T>
__global__ __launch_bounds__(256) void gate_logits_generic(const T *x, const T *Wa, const T *Wb,
                                                           int B, int L, int D, int H,
                                                           float *beta, float *za) {
  const int64_t H2 = 2 * H;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (int64_t)B * L * H2) return;
  const int c = (int)(i % H2);
  const int64_t bt = i / H2;
  const T *xr = x + bt * D;
  const T *wr = c < H ? Wa + (int64_t)c * D : Wb + (int64_t)(c - H) * D;
  float acc = 0.f;
  for (int k = 0; k < D; ++k) acc = fmaf((float)xr[k], (float)wr[k], acc);
  if (c < H)
    za[bt * H + c] = acc;
  else
    beta[bt * H + (c - H)] = sigmoid(acc);
}

// One wavefront per (stream, head): lane j sums partials j, j + 64, ... in
// order, then a fixed butterfly; lane 0's total is the result.
__global__ __launch_bounds__(256) void gate_alpha(const float *za, int B, int H, int L, int nta,
                                                  float *alpha) {
  const int bh = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (bh >= B * H) return;
  const int b = bh / H, h = bh % H;
  const float *src = za + (int64_t)b * nta * H + h;
  float s = 0.f;
  for (int j = lane; j < nta; j += 64) s += src[(int64_t)j * H];
#pragma unroll
  for (int m = 32; m > 0; m >>= 1) s += __shfl_xor(s, m, 64);
  if (lane == 0) alpha[bh] = sigmoid(s / (float)L);
}

}  // namespace

GatePlan plan_gate(int64_t B, int64_t L, int64_t D, int64_t H, int dtype) {
  GatePlan g;
  g.mfma = dtype == 0 && D % kGGroup == 0;
  if (g.mfma) {
    g.ntt = (int)((L + kGTok - 1) / kGTok);
    g.nnt = (int)((2 * H + kGCols - 1) / kGCols);
    g.nta = g.ntt;
  } else {
    g.ntt = g.nnt = 0;
    g.nta = (int)L;
  }
  g.ws_bytes = ((size_t)B * g.nta * H * sizeof(float) + 255) & ~(size_t)255;
  return g;
}

hipError_t launch_gate_projections(const GateArgs &a, hipStream_t s) {
  const GatePlan &g = a.plan;
  float *za = (float *)a.ws;
  if (g.mfma) {
    GateLogitParams p{(const bf16 *)a.x, (const bf16 *)a.Wa, (const bf16 *)a.Wb, a.B, a.L, a.D,
                      a.H, g.ntt, g.nnt, a.beta, za};
    const int64_t blocks = (int64_t)a.B * g.ntt * g.nnt;
    launch(gate_logits_mfma, dim3((unsigned)blocks), dim3(kGWaves * 64), 0, s, p);
  } else {
    const int64_t n = (int64_t)a.B * a.L * 2 * a.H;
    const dim3 grid((unsigned)((n + 255) / 256));
    if (a.dtype == 0)
      launch(gate_logits_generic<bf16>, grid, dim3(256), 0, s, (const bf16 *)a.x,
                         (const bf16 *)a.Wa, (const bf16 *)a.Wb, a.B, a.L, a.D, a.H, a.beta, za);
    else
      launch(gate_logits_generic<float>, grid, dim3(256), 0, s, (const float *)a.x,
                         (const float *)a.Wa, (const float *)a.Wb, a.B, a.L, a.D, a.H, a.beta,
                         za);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t nbh = (int64_t)a.B * a.H;
  launch(gate_alpha, dim3((unsigned)((nbh + 3) / 4)), dim3(256), 0, s, za, a.B, a.H,
                     a.L, g.nta, a.alpha);
  return hipGetLastError();
}

}  // namespace arl2
