// One chunk's contribution to the gated delta state update (bf16 io,
// d = 128), as a device function for the first launch of a clean pass.
//
// Method: "Technical Summary: Attend Locally, Remember Linearly (ARL2)",
// section 2.1 (state update) and section 2.2 (the state is written once per
// frame, after the clean pass, from the pre-update state):
//   K' = L2norm(k W_k), V' = v W_v, R = V' - K' S_{N-1},
//   S_N = alpha S_{N-1} + K'^T diag(beta) R.
// A chunk of 32*NT tokens of one (stream, head) computes
// dS_c = K'_c^T diag(beta_c) R_c into the workspace; the combine launch then
// applies S = alpha S + sum_c dS_c in a fixed chunk order (deterministic, no
// atomics). Every chunk reads the same pre-update S, which no other work of
// its launch writes.
//
// Precision: the feature maps use bf16 operands (the inputs are bf16) with
// fp32 accumulation, which is exact per product. The two products that
// involve the fp32 state or the fp32 K' — K'S and K'^T (beta R) — use the
// split-bf16 scheme (x = hi + lo, three MFMAs hi*hi + hi*lo + lo*hi; Henry,
// Tang and Heinecke, ARITH 2019), about 2^-16 relative per product, because
// plain bf16 operands lose about 2^-9 per frame on the state.
//
// Within a workgroup (4 wavefronts; wavefront w owns state columns
// d_v in [32w, 32w + 32)):
//  (0) W_k and W_v are copied into LDS as swizzled 128x128 tiles; each wave
//      keeps -S[:, its columns] in registers as split-bf16 MFMA operands;
//  (1) wave t < NT computes (k W_k)^T for token tile t (lanes = tokens,
//      registers = d_k), the L2 norms in registers, and writes K' (split
//      bf16, rows = tokens) over the weight tiles;
//  (2) every wave forms R = v W_v - K'S for all tokens of the chunk and its
//      columns (rows = tokens), scales by beta and keeps the result as
//      split-bf16 operands in registers (the accumulator rows line up with
//      the k order of the next product);
//  (3) every wave contracts over the tokens: dS_c[:, its columns] =
//      K'^T (beta R), with K'^T read transposed from LDS.
// No product is computed twice. The 128-row tiles live in two 64-row LDS
// arrays each (the attention kernel's double-buffered key and value tiles),
// so every row index below selects an array by its top bit.
#pragma once

#include "arl2_device.h"

namespace arl2 {

// A 128-row tile of 256-byte rows (tile_off layout) held in two 64-row LDS
// arrays.
struct SplitTile {
  char *lo, *hi;  // rows 0 .. 63, rows 64 .. 127
  __device__ __forceinline__ char *half(int row) const { return row < 64 ? lo : hi; }
};

// tile_col_operand on a split tile: rows k0 .. k0+3 and k1 .. k1+3 must lie
// in the same half.
__device__ __forceinline__ bf16x8 split_col_operand(const SplitTile &t, int k0, int k1, int lane,
                                                    int bb) {
  return tile_col_operand(t.half(k0), k0 & 63, k1 & 63, lane, bb);
}

struct DeltaKParams {
  const bf16 *k, *v, *Wk, *Wv;
  const float *S, *beta;
  int H, L, nchunk, nitems;
  float *ws_dS;
};

// One chunk of 32*NT tokens (item = (stream, head, chunk), chunk fastest).
// A holds W_k, then K' (hi); Bt W_v, then K' (lo).
template <int NT>
__device__ __forceinline__ void delta_body(const DeltaKParams p, int item, SplitTile A,
                                           SplitTile Bt, float *betas) {
  static_assert(NT >= 1 && NT <= 4, "token tiles per chunk");
  constexpr int D = 128;
  constexpr int T = 32 * NT;
  const int chunk = item % p.nchunk;
  const int rest = item / p.nchunk;
  const int h = rest % p.H, b = rest / p.H;

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, hl = lane >> 5, l32 = lane & 31;
  const int t0 = chunk * T;
  const int nvalid = min(T, p.L - t0);
  const int tokB = p.H * D * 2;  // bytes between tokens (H <= 65535)
  const char *kbase = (const char *)(p.k + (((int64_t)b * p.L + t0) * p.H + h) * D);
  const char *vbase = (const char *)(p.v + (((int64_t)b * p.L + t0) * p.H + h) * D);
  // Rows at or past the chunk's last valid token read as zeros.
  const uint32_t span = (uint32_t)nvalid * (uint32_t)tokB;
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(kbase, span);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(vbase, span);

  // (0) Weight tiles: wave w copies 4-row chunks 8w .. 8w+7 of each map
  // (rows 32w .. 32w+31, so one half per wave); lane (r4 = l/16, pos = l%16)
  // fetches unit pos ^ swizzle of its row, so the bytes land in the
  // swizzled layout.
  {
    const bf16 *Wk = p.Wk + (int64_t)h * D * D;
    const bf16 *Wv = p.Wv + (int64_t)h * D * D;
    const int r4 = lane >> 4, pos = lane & 15;
    char *dA = A.half(32 * wave), *dB = Bt.half(32 * wave);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int cc = 8 * wave + i, row = 4 * cc + r4;
      const int off = row * D + 8 * (pos ^ tile_swz(row & 15));
      global_to_lds16(Wk + off, dA + (cc & 15) * 1024);
      global_to_lds16(Wv + off, dB + (cc & 15) * 1024);
    }
  }
  if (tid < T)
    betas[tid] = tid < nvalid ? p.beta[((int64_t)b * p.L + t0 + tid) * p.H + h] : 0.f;

  // -S[d_k][d_v] for d_v = 32*wave + l%32 as B operands, split bf16: group g
  // holds d_k = 16g + 8*(l/32) .. +7.
  bf16x8 snh[8], snl[8];
  {
    const float *Sp = p.S + ((int64_t)b * p.H + h) * D * D + 32 * wave + l32;
#pragma unroll
    for (int g = 0; g < 8; ++g)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        bf16 hi, lo;
        split_bf16(-Sp[(16 * g + 8 * hl + j) * D], hi, lo);
        snh[g][j] = hi;
        snl[g][j] = lo;
      }
  }

  // This wave's token tile (if any) as B operands: lane l holds token
  // 32*wave + l%32, features 16c + 8*(l/32) .. +7.
  bf16x8 kop[8];
  if (wave < NT) {
#pragma unroll
    for (int c = 0; c < 8; ++c)
      kop[c] = buffer_load16(rk, (32 * wave + l32) * tokB + 32 * c + 16 * hl);
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  // (1) (k W_k)^T: rows d_k = 32bb + 8(i/4) + 4(l/32) + i%4, column = token.
  f32x16 kt[4];
  float inv = 0.f;
  if (wave < NT) {
#pragma unroll
    for (int bb = 0; bb < 4; ++bb) kt[bb] = zero16();
    // Four independent chains, interleaved.
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const int k0 = 16 * c + 8 * hl;
      bf16x8 wa[4];
#pragma unroll
      for (int bb = 0; bb < 4; ++bb) wa[bb] = split_col_operand(A, k0, k0 + 4, lane, bb);
#pragma unroll
      for (int bb = 0; bb < 4; ++bb) kt[bb] = mfma32(wa[bb], kop[c], kt[bb]);
    }
    float ss = 0.f;
#pragma unroll
    for (int bb = 0; bb < 4; ++bb)
#pragma unroll
      for (int i = 0; i < 16; ++i) ss = fmaf(kt[bb][i], kt[bb][i], ss);
    ss = halves_sum(ss);
    inv = 1.f / fmaxf(sqrtf(ss), kL2Eps);
  }
  // W_v[d_in][d_v] for this wave's columns as B operands (k = d_in).
  bf16x8 wv[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const int k0 = 16 * c + 8 * hl;
    wv[c] = split_col_operand(Bt, k0, k0 + 4, lane, wave);
  }
  __syncthreads();  // every read of the weight tiles is done

  // K' rows (split bf16) over the weight tiles: row = token, column = d_k.
  if (wave < NT) {
    const int row = 32 * wave + l32;
    char *hA = A.half(row), *hB = Bt.half(row);
#pragma unroll
    for (int bb = 0; bb < 4; ++bb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        bf16x4 th, tl;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          bf16 hi, lo;
          split_bf16(kt[bb][4 * r + e] * inv, hi, lo);
          th[e] = hi;
          tl[e] = lo;
        }
        const int off = tile_off(row & 63, 4 * bb + r) + 8 * hl;
        *(bf16x4 *)(hA + off) = th;
        *(bf16x4 *)(hB + off) = tl;
      }
  }
  __syncthreads();

  // (2) R = v W_v - K'S per token tile, then beta R as split-bf16 B
  // operands: accumulator registers 8*g2 .. 8*g2+7 hold tokens
  // 16*g2 + swap_bits23(8*(l/32) + j) of the tile.
  bf16x8 rh[NT][2], rl[NT][2];
  bf16x8 va[8], vn[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) va[c] = buffer_load16(rv, l32 * tokB + 32 * c + 16 * hl);
#pragma unroll
  for (int tt = 0; tt < NT; ++tt) {
    if (tt + 1 < NT) {
#pragma unroll
      for (int c = 0; c < 8; ++c)
        vn[c] = buffer_load16(rv, (32 * (tt + 1) + l32) * tokB + 32 * c + 16 * hl);
    }
    // Two accumulation chains (v W_v + hi*hi, the two cross terms),
    // alternating so that no MFMA waits on the one just before it.
    const char *kA = tt < 2 ? A.lo : A.hi, *kB = tt < 2 ? Bt.lo : Bt.hi;
    f32x16 a0 = zero16(), a1 = zero16();
#pragma unroll
    for (int g = 0; g < 8; ++g) {
      const int off = tile_off((32 * tt + l32) & 63, 2 * g + hl);
      const bf16x8 ah = *(const bf16x8 *)(kA + off);
      const bf16x8 al = *(const bf16x8 *)(kB + off);
      a0 = mfma32(va[g], wv[g], a0);
      a1 = mfma32(ah, snl[g], a1);
      a0 = mfma32(ah, snh[g], a0);
      a1 = mfma32(al, snh[g], a1);
    }
    f32x16 acc;
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = a0[i] + a1[i];
#pragma unroll
    for (int g2 = 0; g2 < 2; ++g2)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int tok = 32 * tt + 16 * g2 + 8 * (j >> 2) + 4 * hl + (j & 3);
        bf16 hi, lo;
        split_bf16(acc[8 * g2 + j] * betas[tok], hi, lo);
        rh[tt][g2][j] = hi;
        rl[tt][g2][j] = lo;
      }
    if (tt + 1 < NT) {
#pragma unroll
      for (int c = 0; c < 8; ++c) va[c] = vn[c];
    }
  }

  // (3) dS_c[d_k][d_v] = sum over tokens of K'[t][d_k] (beta R)[t][d_v]:
  // A = K'^T read transposed (tokens in the same permuted order).
  f32x16 ds[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) ds[db] = zero16();
#pragma unroll
  for (int tt = 0; tt < NT; ++tt)
#pragma unroll
    for (int g2 = 0; g2 < 2; ++g2) {
      const int k0 = 32 * tt + 16 * g2 + 4 * hl;
      bf16x8 ah[4], al[4];
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        ah[db] = split_col_operand(A, k0, k0 + 8, lane, db);
        al[db] = split_col_operand(Bt, k0, k0 + 8, lane, db);
      }
      // Four independent chains, interleaved.
#pragma unroll
      for (int db = 0; db < 4; ++db) ds[db] = mfma32(ah[db], rh[tt][g2], ds[db]);
#pragma unroll
      for (int db = 0; db < 4; ++db) ds[db] = mfma32(ah[db], rl[tt][g2], ds[db]);
#pragma unroll
      for (int db = 0; db < 4; ++db) ds[db] = mfma32(al[db], rh[tt][g2], ds[db]);
    }

  float *wd = p.ws_dS + (((int64_t)b * p.H + h) * p.nchunk + chunk) * D * D + 32 * wave + l32;
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int dk = 32 * db + 8 * (i >> 2) + 4 * hl + (i & 3);
      wd[dk * D] = ds[db][i];
    }
}

}  // namespace arl2
