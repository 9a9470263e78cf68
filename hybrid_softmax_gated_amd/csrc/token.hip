// Token-level state access: the ablation that frame-level access is compared
// with ("Technical Summary: Attend Locally, Remember Linearly (ARL2)",
// section 4; frame-level access is section 2.2). Inside a frame the tokens
// write the state one after another and each token reads it right after its
// own write:
//   S_1 = alpha S_0 + beta_1 k'_1 (v'_1 - k'_1^T S_0),
//   S_i = S_{i-1} + beta_i k'_i (v'_i - k'_i^T S_{i-1})   (i > 1),
//   O_inter[i] = q'_i S_i.
// The forget gate acts once per frame, with the first token, and the first
// residual reads the ungated state, so a one-token frame is the frame-level
// update. Noisy passes form the within-frame states for their reads only;
// the clean pass keeps S_L.
//
// The recurrence is evaluated in chunks of 64 tokens (the chunked form of
// the delta rule; Yang et al., "Parallelizing Linear Transformers with the
// Delta Rule over Sequence Length", NeurIPS 2024). For a chunk with keys K,
// values V, queries Q and state S entering it:
//   R = T diag(beta g) (V - K S) with T = (I + tril(diag(beta) K K^T, -1))^-1
//     = U - W S,  W = T diag(beta g) K,  U = T diag(beta) V,
//   O = Q S' + tril(Q K^T) R,   S <- S' + K^T R,
// where S' = alpha S and g = (1, alpha, ..., alpha) for the first chunk of
// the frame (S' = S, g = 1 after it). W, U, Q, K^T and M = tril(Q K^T) do
// not depend on S, so:
//   tl_prep_kernel  (one workgroup per stream, head and chunk, all in
//                   parallel): projections, L2 norms, K K^T and Q K^T on the
//                   matrix cores, T by 16 x 16 blocks in fp32, W and U as
//                   T times the right-hand sides on the matrix cores, all
//                   stored as ready-made MFMA operands;
//   tl_recur_kernel (one workgroup per stream, head and 16 state columns):
//                   the chunks in order, S in registers.
// Precision: products that feed the state (K K^T, W S, K^T R) use split
// bf16 (x = hi + lo, three MFMAs; Henry, Tang and Heinecke, ARITH 2019);
// the output-only products (Q K^T's use in O, Q S, M R) take Q and M in
// plain bf16. T is formed in fp32; T times the right-hand sides uses split
// bf16.
#include "arl2_device.h"
#include "arl2_kernels.h"

#include <math.h>

namespace arl2 {
namespace {

constexpr int D = 128;
constexpr int TC = kTokenChunk;  // tokens per chunk (64)
constexpr int NSL = D / 16;      // 16-column state slices per head
constexpr int VROW = D + 4;      // padded fp32 row of a token vector in LDS
constexpr int GROW = TC + 4;     // padded fp32 row of a chunk's Gram matrix

// Chunk record (one per stream, head and chunk), all MFMA-ready, 16 bytes
// per lane with the lane index fastest, so that each wavefront load or store
// covers 1 KB of consecutive bytes:
//   W   [wave 4][row tile 4][hi, lo][lane 64]    bf16x8  (A of W S)
//   Q   [wave 4][row tile 4][lane 64]            bf16x8  (A of Q S)
//   KT  [wave 4][tile 2][kstep 2][hi, lo][lane]  bf16x8  (A of K^T R)
//   M   [row tile 4][kstep 2][lane 64]           bf16x8  (A of M R)
//   U   [row tile 4][slice 8][lane 64]           f32x4   (R layout)
constexpr int OFF_W = 0;
constexpr int OFF_Q = OFF_W + 4 * 64 * 4 * 32;
constexpr int OFF_KT = OFF_Q + 4 * 64 * 4 * 16;
constexpr int OFF_M = OFF_KT + 4 * 64 * 2 * 2 * 32;
constexpr int OFF_U = OFF_M + 4 * 64 * 2 * 16;
constexpr int REC = OFF_U + 4 * NSL * 64 * 16;
static_assert(REC == kTokenRecordBytes, "chunk record size");

// The k order of every MFMA operand below. With the 16x16x32 layout an
// accumulator tile gives lane l rows 4(l/16) + i (i < 4); operand position
// 8(l/16) + e of a 32-deep step is fed from rows pi(l/16, e) of two
// consecutive tiles, so accumulators become operands without moving data.
__device__ __forceinline__ constexpr int pi32(int g, int e) {
  return e < 4 ? 4 * g + e : 16 + 4 * g + (e - 4);
}

__device__ __forceinline__ void split8(const float *x, bf16x8 &hi, bf16x8 &lo) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    bf16 h, l;
    split_bf16(x[e], h, l);
    hi[e] = h;
    lo[e] = l;
  }
}

// ------------------------------------------------------------------ prep
struct PrepParams {
  const bf16 *q, *k, *v;       // [B][L][H][128]
  const bf16 *Wq, *Wk, *Wv;    // [H][128][128]
  const float *alpha, *beta;   // [B][H], [B][L][H]
  int H, L, nchunk, nitems, per_xcd;
  char *rec;                   // [B][H][nchunk] records
};

// Eight wavefronts. (A) waves 0-5 each project one 32-token tile of one map
// (k, v, q); (B) waves 0-5 each form one 32x32 tile of K K^T or Q K^T while
// waves 6-7 write the Q and K^T records; (C) T = (I + A)^-1 by 16 x 16
// blocks while waves 4-7 write the M record, then W and U = T x (right-hand
// sides) on the matrix cores; (D) everyone writes the W and U records.
__global__ __launch_bounds__(512) void tl_prep_kernel(PrepParams p) {
  __shared__ __attribute__((aligned(16))) float vecs[3][TC][VROW];  // Q', K', V' (then W, U)
  __shared__ __attribute__((aligned(16))) float gram[2][TC][GROW];  // beta-scaled K K^T, Q K^T
  __shared__ __attribute__((aligned(16))) float tinv[TC][GROW];     // T = (I + A)^-1
  __shared__ float betas[TC], bgs[TC];
  const int bid = blockIdx.x;
  const int item = (bid & 7) * p.per_xcd + (bid >> 3);
  if (item >= p.nitems) return;
  const int chunk = item % p.nchunk;
  const int bh = item / p.nchunk;
  const int h = bh % p.H, b = bh / p.H;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, hl = lane >> 5, l32 = lane & 31;
  const int g = lane >> 4, r16 = lane & 15;
  // T's strict upper part stays zero (its blocks on and below the diagonal
  // are written in phase C).
  for (int e = tid; e < TC * GROW; e += 512) (&tinv[0][0])[e] = 0.f;
  const int t0 = chunk * TC;
  const int nvalid = min(TC, p.L - t0);
  const int tokB = p.H * D * 2;
  const float alpha = p.alpha[bh];

  // (A) projections. The three weight tiles sit where the vectors will go.
  char *tiles = (char *)&vecs[0][0][0];
  {
    const bf16 *Ws[3] = {p.Wq + (int64_t)h * D * D, p.Wk + (int64_t)h * D * D,
                         p.Wv + (int64_t)h * D * D};
    const int r4 = lane >> 4, pos = lane & 15;
#pragma unroll
    for (int m = 0; m < 3; ++m)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int cc = 4 * wave + i, row = 4 * cc + r4;
        global_to_lds16(Ws[m] + row * D + 8 * (pos ^ tile_swz(row & 15)),
                        tiles + m * 32768 + cc * 1024);
      }
  }
  if (tid < TC) {
    const float bt = tid < nvalid ? p.beta[((int64_t)b * p.L + t0 + tid) * p.H + h] : 0.f;
    betas[tid] = bt;
    bgs[tid] = (chunk == 0 && tid > 0) ? bt * alpha : bt;
  }
  // Projection job of waves 0-5: map k, v, q for waves (0, 1), (2, 3),
  // (4, 5); token tile wave & 1.
  const bool proj = wave < 6;
  const int tt = wave & 1;
  const int m0 = wave < 2 ? 1 : wave < 4 ? 2 : 0;
  bf16x8 op0[8];
  if (proj) {
    const bf16 *src = m0 == 1 ? p.k : m0 == 2 ? p.v : p.q;
    const char *base = (const char *)(src + (((int64_t)b * p.L + t0) * p.H + h) * D);
    const __amdgpu_buffer_rsrc_t r = make_rsrc(base, (uint32_t)nvalid * (uint32_t)tokB);
#pragma unroll
    for (int c = 0; c < 8; ++c) op0[c] = buffer_load16(r, (32 * tt + l32) * tokB + 32 * c + 16 * hl);
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  // (x W)^T: rows = output features 32bb + 8(i/4) + 4(l/32) + i%4, column =
  // token 32 tt + l%32.
  f32x16 a0[4];
  float s0 = 1.f;
  if (proj) {
#pragma unroll
    for (int bb = 0; bb < 4; ++bb) a0[bb] = zero16();
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const int k0 = 16 * c + 8 * hl;
      bf16x8 wa[4];
#pragma unroll
      for (int bb = 0; bb < 4; ++bb)
        wa[bb] = tile_col_operand(tiles + m0 * 32768, k0, k0 + 4, lane, bb);
#pragma unroll
      for (int bb = 0; bb < 4; ++bb) a0[bb] = mfma32(wa[bb], op0[c], a0[bb]);
    }
    if (m0 != 2) {
      float ss = 0.f;
#pragma unroll
      for (int bb = 0; bb < 4; ++bb)
#pragma unroll
        for (int i = 0; i < 16; ++i) ss = fmaf(a0[bb][i], a0[bb][i], ss);
      ss = halves_sum(ss);
      s0 = 1.f / fmaxf(sqrtf(ss), kL2Eps);
    }
  }
  __syncthreads();  // every wave is done with the weight tiles
  if (proj) {
    const int tok = 32 * tt + l32;
#pragma unroll
    for (int bb = 0; bb < 4; ++bb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        f32x4 x;
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = a0[bb][4 * r + e] * s0;
        *(f32x4 *)&vecs[m0][tok][32 * bb + 8 * r + 4 * hl] = x;
      }
  }
  __syncthreads();

  char *rec = p.rec + (int64_t)item * REC;
  if (proj) {
    // (B) tile `wave` of: G00 G10 G11 (K K^T) and P00 P10 P11 (Q K^T), split
    // bf16. Rows are tokens 32rb + 8(i/4) + 4(l/32) + i%4, columns tokens
    // 32cb + l%32.
    const int mat = wave >= 3 ? 1 : 0, idx = wave % 3;
    const int rb = idx == 0 ? 0 : 1, cb = idx == 2 ? 1 : 0;
    const float(*A)[VROW] = vecs[mat == 0 ? 1 : 0];
    f32x16 acc = zero16();
#pragma unroll
    for (int st = 0; st < 8; ++st) {
      const int f = 16 * st + 8 * hl;
      float xa[8], xb[8];
      *(f32x4 *)&xa[0] = *(const f32x4 *)&A[32 * rb + l32][f];
      *(f32x4 *)&xa[4] = *(const f32x4 *)&A[32 * rb + l32][f + 4];
      *(f32x4 *)&xb[0] = *(const f32x4 *)&vecs[1][32 * cb + l32][f];
      *(f32x4 *)&xb[4] = *(const f32x4 *)&vecs[1][32 * cb + l32][f + 4];
      bf16x8 ah, al, bh8, bl8;
      split8(xa, ah, al);
      split8(xb, bh8, bl8);
      acc = mfma32(ah, bh8, acc);
      acc = mfma32(ah, bl8, acc);
      acc = mfma32(al, bh8, acc);
    }
    // P is stored as is; K K^T transposed and with column i scaled by
    // beta_i, i.e. gram[0][j][i] = beta_i (k'_i . k'_j), the row the
    // substitution below reads for token j.
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int ri = 32 * rb + 8 * (i >> 2) + 4 * hl + (i & 3), cj = 32 * cb + l32;
      if (mat == 0)
        gram[0][cj][ri] = betas[ri] * acc[i];
      else
        gram[1][ri][cj] = acc[i];
    }
  } else {
    // Q (plain bf16) and K^T (split) records, straight from the vectors;
    // waves 6 and 7 each take two of the four d_k blocks.
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2) {
      const int w = (wave - 6) + 2 * k2;
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) {
        const float *row = &vecs[0][16 * rt + r16][32 * w + 4 * g];
        bf16x8 qh;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          qh[e] = (bf16)row[e];
          qh[4 + e] = (bf16)row[16 + e];
        }
        *(bf16x8 *)(rec + OFF_Q + (w * 4 + rt) * 1024 + lane * 16) = qh;
      }
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          float x[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) x[e] = vecs[1][32 * ks + pi32(g, e)][32 * w + 16 * t + r16];
          bf16x8 hi, lo;
          split8(x, hi, lo);
          char *dst = rec + OFF_KT + ((w * 2 + t) * 2 + ks) * 2048 + lane * 16;
          *(bf16x8 *)dst = hi;
          *(bf16x8 *)(dst + 1024) = lo;
        }
    }
  }
  __syncthreads();

  // (C) W = T diag(beta g) K and U = T diag(beta) V with
  // T = (I + A)^-1, A = tril(diag(beta) K K^T, -1) (unit lower triangular),
  // built from 16 x 16 blocks in fp32: the diagonal blocks by forward
  // substitution, then the blocks below them one sub-diagonal at a time,
  //   T_IJ = -T_II sum_{J <= K < I} A_IK T_KJ,
  // and finally X = T [diag(beta g) K | diag(beta) V] on the matrix cores
  // (split bf16). Waves 4-7 write the M = tril(Q K^T) record meanwhile.
  // A[i][j] is read as gram[0][j][i].
  if (wave == 0) {
    // Diagonal block I = lane / 16, column c = lane % 16, column order.
    const int I = lane >> 4, c = lane & 15, o = 16 * I;
    float t[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) t[r] = r == c ? 1.f : 0.f;
#pragma unroll
    for (int j = 0; j < 15; ++j) {
      float a[16];
#pragma unroll
      for (int r4 = 0; r4 < 16; r4 += 4) *(f32x4 *)&a[r4] = *(const f32x4 *)&gram[0][o + j][o + r4];
#pragma unroll
      for (int r = j + 1; r < 16; ++r) t[r] = fmaf(-a[r], t[j], t[r]);
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) tinv[o + r][o + c] = t[r];
  } else if (wave >= 4) {
    const int rt = wave - 4, i = 16 * rt + r16;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      bf16x8 mh;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int j = 32 * ks + pi32(g, e);
        mh[e] = (bf16)(j <= i ? gram[1][i][j] : 0.f);
      }
      *(bf16x8 *)(rec + OFF_M + (rt * 2 + ks) * 1024 + lane * 16) = mh;
    }
  }
  __syncthreads();
  // Sub-diagonal d = 1, 2, 3: wave J < 4 - d forms block (J + d, J). Lane
  // (r = l / 4, c4 = l % 4) owns row r, columns 4c4 .. 4c4+3 of the block.
#pragma unroll
  for (int dgl = 1; dgl < 4; ++dgl) {
    if (wave < 4 - dgl) {
      const int J = wave, I = J + dgl, r = lane >> 2, c4 = lane & 3;
      // P = sum_{J <= K < I} A_IK T_KJ, row r.
      f32x4 pr = {0.f, 0.f, 0.f, 0.f};
      for (int K = J; K < I; ++K) {
#pragma unroll
        for (int k = 0; k < 16; ++k) {
          const float a = gram[0][16 * K + k][16 * I + r];
          const f32x4 tk = *(const f32x4 *)&tinv[16 * K + k][16 * J + 4 * c4];
#pragma unroll
          for (int e = 0; e < 4; ++e) pr[e] = fmaf(a, tk[e], pr[e]);
        }
      }
      // The block's own slot holds P until every lane has read what it needs.
      *(f32x4 *)&tinv[16 * I + r][16 * J + 4 * c4] = pr;
      __builtin_amdgcn_s_waitcnt(0xC07F);
      __builtin_amdgcn_wave_barrier();
      f32x4 res = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        const float tik = tinv[16 * I + r][16 * I + k];
        const f32x4 pk = *(const f32x4 *)&tinv[16 * I + k][16 * J + 4 * c4];
#pragma unroll
        for (int e = 0; e < 4; ++e) res[e] = fmaf(-tik, pk[e], res[e]);
      }
      __builtin_amdgcn_s_waitcnt(0xC07F);
      __builtin_amdgcn_wave_barrier();
      *(f32x4 *)&tinv[16 * I + r][16 * J + 4 * c4] = res;
    }
    __syncthreads();
  }
  {
    // X = T RHS: wave w takes columns 32w .. 32w+31 of [K | V] (K for
    // w < 4), rows in two 32-row tiles, k in four steps of 16.
    const int m = wave < 4 ? 1 : 2, col = 32 * (wave & 3) + l32;
    float(*X)[VROW] = vecs[m];
    const float *coef = wave < 4 ? bgs : betas;
    f32x16 acc[2] = {zero16(), zero16()};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int k0 = 16 * ks + 8 * hl;
      float xb[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) xb[e] = X[k0 + e][col] * coef[k0 + e];
      bf16x8 bh8, bl8;
      split8(xb, bh8, bl8);
#pragma unroll
      for (int rt = 0; rt < 2; ++rt) {
        float xa[8];
        *(f32x4 *)&xa[0] = *(const f32x4 *)&tinv[32 * rt + l32][k0];
        *(f32x4 *)&xa[4] = *(const f32x4 *)&tinv[32 * rt + l32][k0 + 4];
        bf16x8 ah, al;
        split8(xa, ah, al);
        acc[rt] = mfma32(ah, bh8, acc[rt]);
        acc[rt] = mfma32(ah, bl8, acc[rt]);
        acc[rt] = mfma32(al, bh8, acc[rt]);
      }
    }
    // Every read of this wave's columns is done (the values above fed the
    // MFMAs); the results replace them.
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
      for (int i = 0; i < 16; ++i) X[32 * rt + 8 * (i >> 2) + 4 * hl + (i & 3)][col] = acc[rt][i];
  }
  __syncthreads();

  // (D) W (split) and U records.
#pragma unroll
  for (int k2 = 0; k2 < 2; ++k2) {
    const int combo = 2 * wave + k2, w = combo >> 2, rt = combo & 3;
    const float *row = &vecs[1][16 * rt + r16][32 * w + 4 * g];
    float x[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[e] = row[e];
      x[4 + e] = row[16 + e];
    }
    bf16x8 hi, lo;
    split8(x, hi, lo);
    char *dst = rec + OFF_W + (w * 4 + rt) * 2048 + lane * 16;
    *(bf16x8 *)dst = hi;
    *(bf16x8 *)(dst + 1024) = lo;
  }
#pragma unroll
  for (int k2 = 0; k2 < 4; ++k2) {
    const int unit = tid + 512 * k2;  // (rt, slice, lane)
    const int ln = unit & 63, sl = (unit >> 6) & 7, rt = unit >> 9;
    const int gg = ln >> 4, c = 16 * sl + (ln & 15);
    f32x4 u;
#pragma unroll
    for (int e = 0; e < 4; ++e) u[e] = vecs[2][16 * rt + 4 * gg + e][c];
    *(f32x4 *)(rec + OFF_U + unit * 16) = u;
  }
}

// ------------------------------------------------------------- recurrence
struct RecurParams {
  const char *rec;      // [B][H][nchunk] records
  const float *alpha;   // [B][H]
  float *S;             // [B][H][128][128]
  float *o_inter;       // [B][L][H][128]
  int H, L, nchunk, nitems, per_xcd, update;
};

// Barrier that waits only for LDS traffic, so that global loads of the next
// chunk's operands stay in flight across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

struct ChunkOps {
  bf16x8 wh[4], wl[4], qh[4], kh[2][2], kl[2][2], mh[2];
  f32x4 u;
};

__device__ __forceinline__ void load_ops(ChunkOps &o, const char *rec, int wave, int lane,
                                         int slice) {
  const char *w = rec + OFF_W + wave * 4 * 2048 + lane * 16;
#pragma unroll
  for (int rt = 0; rt < 4; ++rt) {
    o.wh[rt] = *(const bf16x8 *)(w + rt * 2048);
    o.wl[rt] = *(const bf16x8 *)(w + rt * 2048 + 1024);
    o.qh[rt] = *(const bf16x8 *)(rec + OFF_Q + (wave * 4 + rt) * 1024 + lane * 16);
  }
  const char *kt = rec + OFF_KT + wave * 4 * 2048 + lane * 16;
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      o.kh[t][ks] = *(const bf16x8 *)(kt + (2 * t + ks) * 2048);
      o.kl[t][ks] = *(const bf16x8 *)(kt + (2 * t + ks) * 2048 + 1024);
    }
#pragma unroll
  for (int ks = 0; ks < 2; ++ks)
    o.mh[ks] = *(const bf16x8 *)(rec + OFF_M + (wave * 2 + ks) * 1024 + lane * 16);
  o.u = *(const f32x4 *)(rec + OFF_U + ((wave * NSL + slice) * 64 + lane) * 16);
}

struct RecurCtx {
  f32x4 (*red)[2][4][4][64];  // [buf][R/O][wave][tile][lane]
  bf16x8 (*rb)[4][64];         // [buf][tile][lane]: 4 hi, 4 lo
  float *o_inter;
  int H, L, b, h, slice, wave, lane, g, r16;
  float alpha;
};

// One chunk: R = U - W S and Q S from the four waves' shares, then O and
// S <- S' + K^T R (S' = alpha S for the frame's first chunk).
__device__ __forceinline__ void recur_chunk(const RecurCtx &x, const ChunkOps &cur, int c,
                                            f32x4 (&st)[2]) {
  const int wave = x.wave, lane = x.lane, g = x.g, r16 = x.r16;
  const float alpha = x.alpha;
  auto &red = x.red;
  auto &rb = x.rb;
  const int buf = c & 1;
  // S rows of this wave as a 32-deep B operand (k order pi32).
  float sv[8];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    sv[e] = st[0][e];
    sv[4 + e] = st[1][e];
  }
  bf16x8 sh, sl;
  split8(sv, sh, sl);
#pragma unroll
  for (int rt = 0; rt < 4; ++rt) {
    f32x4 pr = mfma16(cur.wh[rt], sh, zero4());
    pr = mfma16(cur.wh[rt], sl, pr);
    pr = mfma16(cur.wl[rt], sh, pr);
    f32x4 po = mfma16(cur.qh[rt], sh, zero4());
    po = mfma16(cur.qh[rt], sl, po);
    red[buf][0][wave][rt][lane] = pr;
    red[buf][1][wave][rt][lane] = po;
  }
  lds_barrier();
  // Row tile `wave` of R = U - W S and of Q S (summed in wave order).
  f32x4 r = cur.u, o = zero4();
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const f32x4 a = red[buf][0][w][wave][lane], q = red[buf][1][w][wave][lane];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      r[e] -= a[e];
      o[e] += q[e];
    }
  }
  if (c == 0) {
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] *= alpha;
  }
  {
    bf16x8 t;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      bf16 hi, lo;
      split_bf16(r[e], hi, lo);
      t[e] = hi;
      t[4 + e] = lo;
    }
    rb[buf][wave][lane] = t;
  }
  lds_barrier();
  // R as 32-deep B operands over the chunk's tokens (k order pi32).
  bf16x8 rh[2], rl[2];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    const bf16x8 a = rb[buf][2 * ks][lane], z = rb[buf][2 * ks + 1][lane];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      rh[ks][e] = a[e];
      rh[ks][4 + e] = z[e];
      rl[ks][e] = a[4 + e];
      rl[ks][4 + e] = z[4 + e];
    }
  }
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    o = mfma16(cur.mh[ks], rh[ks], o);
    o = mfma16(cur.mh[ks], rl[ks], o);
  }
  {
    const int tok0 = c * TC + 16 * wave + 4 * g;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (tok0 + e < x.L)
        x.o_inter[(((int64_t)x.b * x.L + tok0 + e) * x.H + x.h) * D + 16 * x.slice + r16] = o[e];
  }
  if (c == 0) {
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e) st[t][e] *= alpha;
  }
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      st[t] = mfma16(cur.kh[t][ks], rh[ks], st[t]);
      st[t] = mfma16(cur.kh[t][ks], rl[ks], st[t]);
      st[t] = mfma16(cur.kl[t][ks], rh[ks], st[t]);
    }
}

// Wavefront w keeps rows 32w .. 32w+31 (d_k) of the slice's 16 columns of S
// as two accumulator tiles; it forms its share of W S and Q S, reduces row
// tile w of R and O over the four shares, and updates its rows with K^T R.
// The operands of chunk c + 2 are loaded while chunk c runs (three register
// sets in turn, so no set is copied and no load is waited for early).
__global__ __launch_bounds__(256, 1) void tl_recur_kernel(RecurParams p) {
  __shared__ __attribute__((aligned(16))) f32x4 red[2][2][4][4][64];
  __shared__ __attribute__((aligned(16))) bf16x8 rb[2][4][64];
  const int bid = blockIdx.x;
  const int item = (bid & 7) * p.per_xcd + (bid >> 3);
  if (item >= p.nitems) return;
  const int slice = item % NSL;
  const int bh = item / NSL;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, g = lane >> 4, r16 = lane & 15;
  float *Sh = p.S + (int64_t)bh * D * D + 16 * slice + r16;
  f32x4 st[2];
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i) st[t][i] = Sh[(32 * wave + 16 * t + 4 * g + i) * D];
  const RecurCtx x{red, rb, p.o_inter, p.H, p.L, bh / p.H, bh % p.H, slice, wave, lane, g, r16,
                   p.alpha[bh]};
  const char *rec0 = p.rec + (int64_t)bh * p.nchunk * REC;
  const int n = p.nchunk;
  ChunkOps A, B, C;
  load_ops(A, rec0, wave, lane, slice);
  if (n > 1) load_ops(B, rec0 + REC, wave, lane, slice);
  for (int c = 0; c < n; c += 3) {
    if (c + 2 < n) load_ops(C, rec0 + (int64_t)(c + 2) * REC, wave, lane, slice);
    recur_chunk(x, A, c, st);
    if (c + 1 >= n) break;
    if (c + 3 < n) load_ops(A, rec0 + (int64_t)(c + 3) * REC, wave, lane, slice);
    recur_chunk(x, B, c + 1, st);
    if (c + 2 >= n) break;
    if (c + 4 < n) load_ops(B, rec0 + (int64_t)(c + 4) * REC, wave, lane, slice);
    recur_chunk(x, C, c + 2, st);
  }
  if (p.update) {
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) Sh[(32 * wave + 16 * t + 4 * g + i) * D] = st[t][i];
  }
}

// ---------------------------------------------------------------- generic
__device__ __forceinline__ float ldv(const float *p) { return *p; }
__device__ __forceinline__ float ldv(const bf16 *p) { return (float)*p; }
__device__ __forceinline__ void stv(float *p, float x) { *p = x; }
__device__ __forceinline__ void stv(bf16 *p, float x) { *p = (bf16)x; }

// Any dtype, d in {16, 128}: one workgroup of d threads per (stream, head),
// the tokens strictly in order; thread n keeps column n of S in registers.
// Writes out = O_intra + O_inter directly.
template <typename T, int Dm>
__global__ __launch_bounds__(Dm) void tl_generic_kernel(const T *q, const T *k, const T *v,
                                                        const T *W, const float *o_intra,
                                                        float *S, const float *alpha,
                                                        const float *beta, int H, int L,
                                                        int update, T *out) {
  __shared__ float xs[3][Dm];  // q, k, v of the token
  __shared__ float ps[3][Dm];  // q', k', v'
  __shared__ float nrm[2];
  const int n = threadIdx.x, h = blockIdx.x, b = blockIdx.y;
  const int bh = b * H + h;
  const T *Wq = W + (int64_t)h * Dm * Dm;
  const T *Wk = W + ((int64_t)H + h) * Dm * Dm;
  const T *Wv = W + ((int64_t)2 * H + h) * Dm * Dm;
  float *Sh = S + (int64_t)bh * Dm * Dm;
  float s[Dm];
#pragma unroll
  for (int m = 0; m < Dm; ++m) s[m] = Sh[m * Dm + n];
  const float a = alpha[bh];
  for (int i = 0; i < L; ++i) {
    const int64_t row = (((int64_t)b * L + i) * H + h) * Dm;
    xs[0][n] = ldv(q + row + n);
    xs[1][n] = ldv(k + row + n);
    xs[2][n] = ldv(v + row + n);
    __syncthreads();
    float pq = 0.f, pk = 0.f, pv = 0.f;
    for (int m = 0; m < Dm; ++m) {
      pq = fmaf(xs[0][m], ldv(Wq + m * Dm + n), pq);
      pk = fmaf(xs[1][m], ldv(Wk + m * Dm + n), pk);
      pv = fmaf(xs[2][m], ldv(Wv + m * Dm + n), pv);
    }
    ps[0][n] = pq;
    ps[1][n] = pk;
    ps[2][n] = pv;
    __syncthreads();
    if (n < 2) {
      float ss = 0.f;
      for (int m = 0; m < Dm; ++m) ss = fmaf(ps[n][m], ps[n][m], ss);
      nrm[n] = 1.f / fmaxf(sqrtf(ss), kL2Eps);
    }
    __syncthreads();
    const float iq = nrm[0], ik = nrm[1];
    float ks = 0.f;
#pragma unroll
    for (int m = 0; m < Dm; ++m) ks = fmaf(ps[1][m] * ik, s[m], ks);
    const float r = beta[((int64_t)b * L + i) * H + h] * (ps[2][n] - ks);
    const float g = i == 0 ? a : 1.f;
    float o = 0.f;
#pragma unroll
    for (int m = 0; m < Dm; ++m) {
      s[m] = fmaf(ps[1][m] * ik, r, g * s[m]);
      o = fmaf(ps[0][m] * iq, s[m], o);
    }
    const float oi = o_intra[((int64_t)bh * L + i) * Dm + n];
    stv(out + row + n, oi + o);
    __syncthreads();
  }
  if (update) {
#pragma unroll
    for (int m = 0; m < Dm; ++m) Sh[m * Dm + n] = s[m];
  }
}

template <typename T, int Dm>
hipError_t tl_generic(const void *q, const void *k, const void *v, const void *W,
                      const float *o_intra, float *S, const float *alpha, const float *beta,
                      int B, int H, int L, int update, void *out, hipStream_t s) {
  launch((tl_generic_kernel<T, Dm>), dim3((unsigned)H, (unsigned)B), dim3(Dm), 0, s,
                     (const T *)q, (const T *)k, (const T *)v, (const T *)W, o_intra, S, alpha,
                     beta, H, L, update, (T *)out);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_token_level_bf16(const TokenLevelArgs &a, hipStream_t s) {
  const int nchunk = (a.L + TC - 1) / TC;
  {
    const int nitems = a.B * a.H * nchunk;
    const int per_xcd = (nitems + 7) / 8;
    PrepParams pp{(const bf16 *)a.q, (const bf16 *)a.k, (const bf16 *)a.v,
                  (const bf16 *)a.Wq, (const bf16 *)a.Wk, (const bf16 *)a.Wv,
                  a.alpha, a.beta, a.H, a.L, nchunk, nitems, per_xcd, (char *)a.records};
    launch(tl_prep_kernel, dim3((unsigned)(8 * per_xcd)), dim3(512), 0, s, pp);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int nitems = a.B * a.H * NSL;
  const int per_xcd = (nitems + 7) / 8;
  RecurParams rp{(const char *)a.records, a.alpha, a.S, a.o_inter, a.H, a.L, nchunk, nitems,
                 per_xcd, a.update};
  launch(tl_recur_kernel, dim3((unsigned)(8 * per_xcd)), dim3(256), 0, s, rp);
  return hipGetLastError();
}

#define ARL2_TL_DISPATCH(...)                                              \
  do {                                                                     \
    if (dtype == 1 && d == 16) return tl_generic<float, 16>(__VA_ARGS__);  \
    if (dtype == 1 && d == 128) return tl_generic<float, 128>(__VA_ARGS__); \
    if (dtype == 0 && d == 16) return tl_generic<bf16, 16>(__VA_ARGS__);   \
    if (dtype == 0 && d == 128) return tl_generic<bf16, 128>(__VA_ARGS__); \
    return hipErrorInvalidValue;                                           \
  } while (0)

hipError_t launch_token_level_generic(int dtype, int d, const void *q, const void *k,
                                      const void *v, const void *W, const float *o_intra,
                                      float *S, const float *alpha, const float *beta, int B,
                                      int H, int L, int update, void *out, hipStream_t s) {
  ARL2_TL_DISPATCH(q, k, v, W, o_intra, S, alpha, beta, B, H, L, update, out, s);
}

}  // namespace arl2
