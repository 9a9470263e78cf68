// The work after the attention kernel in one pass: the combine (merge of
// the attention partials, the inter-frame read and the output), and on the
// clean pass the gated delta state update. Both only read the state, so
// they share one launch; a last kernel applies the update in place.
//
// Gated delta state update of the inter-frame branch (bf16 io, d = 128):
//
// Method: "Technical Summary: Attend Locally, Remember Linearly (ARL2)",
// section 2.1 (state update) and section 2.2 (the state is written once per
// frame, after the clean pass, from the pre-update state):
//   K' = L2norm(k W_k), V' = v W_v, R = V' - K' S_{N-1},
//   S_N = alpha S_{N-1} + K'^T diag(beta) R.
//
// Work split: one workgroup per chunk of 32*NT tokens of one (stream, head)
// computes that chunk's contribution dS_c = K'_c^T diag(beta_c) R_c into the
// workspace; delta_apply_kernel then applies S = alpha S + sum_c dS_c in a
// fixed chunk order (deterministic, no atomics). Every workgroup of the
// first launch reads the same pre-update S, so the in-place write is safe.
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
// No product is computed twice; LDS holds 64 KB, so two workgroups share a
// compute unit.
#include "arl2_device.h"
#include "arl2_kernels.h"

#include <math.h>

namespace arl2 {
namespace {

constexpr int D = 128;
constexpr int TILE_BYTES = D * D * 2;  // one 128-row bf16 tile, 32 KB

struct CombineKParams {
  const char *ws_o;
  const float *ws_ml;
  const bf16 *q, *Wq;  // Wq null: no inter-frame read (plain attention)
  const float *S;
  int H, L, nqblk, nsplit, nitems;
  bf16 *out;
  const float *o_inter;  // [B][L][H][128] fp32, added when set (and Wq null)
};

// out = (sum_s w_s Ohat_s) / (sum_s w_s) + O_inter with w_s = 2^(m_s - M) l_s,
// Ohat_s = O_s / l_s the normalised partial of key range s and M the largest
// m_s. Lanes own queries and registers own d_v, as in the attention
// kernel's accumulators, so the partials are read in the order they were
// written and O_inter comes out of the MFMAs in the same layout.
// Every load is issued before any arithmetic: the state rows (converted to
// bf16 into LDS first, which frees their registers), W_q, the queries, the
// merge weights and the first kPre key ranges' partials. The merge runs
// first and the inter-frame read's last product accumulates onto it.
// Wt: 32 KB of LDS for W_q[h], then the output rows; St: 32 KB for bf16(S).
__device__ __forceinline__ void combine_body(const CombineKParams p, int item, char *Wt,
                                             char *St) {
  const int qblk = item % p.nqblk;
  const int bh = item / p.nqblk;
  const int h = bh % p.H, b = bh / p.H;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, hl = lane >> 5, l32 = lane & 31;
  const int64_t tok = (int64_t)p.H * D;
  const int qrow = qblk * kQBlock + wave * 32 + l32;
  const bool inter = p.Wq != nullptr;

  // State rows (fp32) and W_q[h] (straight into LDS, swizzled).
  f32x4 sx[8][2];
  bf16x8 qop[8];
  if (inter) {
    const float *Sh = p.S + ((int64_t)b * p.H + h) * D * D;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int row = (tid >> 4) + 16 * i, u = tid & 15;
      sx[i][0] = *(const f32x4 *)(Sh + row * D + 8 * u);
      sx[i][1] = *(const f32x4 *)(Sh + row * D + 8 * u + 4);
    }
    const bf16 *W = p.Wq + (int64_t)h * D * D;
    const int r4 = lane >> 4, pos = lane & 15;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int cc = 8 * wave + i, row = 4 * cc + r4;
      global_to_lds16(W + row * D + 8 * (pos ^ tile_swz(row & 15)), Wt + cc * 1024);
    }
    // The wave's 32 queries as B operands: lane l holds query l%32,
    // features 16c + 8*(l/32) .. +7 (zeros past the frame).
    if (qrow < p.L) {
      const bf16 *qp = p.q + ((int64_t)b * p.L + qrow) * tok + (int64_t)h * D + 8 * hl;
#pragma unroll
      for (int c = 0; c < 8; ++c) qop[c] = *(const bf16x8 *)(qp + 16 * c);
    } else {
#pragma unroll
      for (int c = 0; c < 8; ++c) qop[c] = zero_bf16x8();
    }
  }

  // Merge weights of the key ranges for this lane's query, and the first
  // kPre ranges' partials (16-byte units in the order the attention kernel
  // wrote them); further ranges stream through the same registers.
  const int64_t blk0 = (int64_t)item * p.nsplit;
  const int qi = wave * 32 + l32;
  float mv[kMaxSplit], lv[kMaxSplit];
#pragma unroll
  for (int s = 0; s < kMaxSplit; ++s)
    if (s < p.nsplit) {
      const float *ml = p.ws_ml + (blk0 + s) * kPartialML + 2 * qi;
      mv[s] = ml[0];
      lv[s] = ml[1];
    }
  const char *src = p.ws_o + blk0 * kPartialOBytes + (wave * 8 * 64 + lane) * 16;
  constexpr int kPre = 3;
  bf16x8 pr[kPre][8];
#pragma unroll
  for (int s = 0; s < kPre; ++s)
    if (s < p.nsplit) {
#pragma unroll
      for (int u = 0; u < 8; ++u)
        pr[s][u] = *(const bf16x8 *)(src + s * kPartialOBytes + u * 64 * 16);
    }

  if (inter) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int row = (tid >> 4) + 16 * i, u = tid & 15;
      bf16x8 t;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        t[e] = (bf16)sx[i][0][e];
        t[4 + e] = (bf16)sx[i][1][e];
      }
      *(bf16x8 *)(St + tile_off(row, u)) = t;
    }
  }

  float M = -INFINITY;
#pragma unroll
  for (int s = 0; s < kMaxSplit; ++s)
    if (s < p.nsplit) M = fmaxf(M, mv[s]);
  float Lt = 0.f;
#pragma unroll
  for (int s = 0; s < kMaxSplit; ++s)
    if (s < p.nsplit) {
      lv[s] *= exp2_fast(mv[s] - M);
      Lt += lv[s];
    }
  const float il = 1.f / Lt;
  // acc = sum_s (w_s / sum w) Ohat_s, range by range in range order.
  f32x16 acc[4];
#pragma unroll
  for (int bb = 0; bb < 4; ++bb) acc[bb] = zero16();
#pragma unroll
  for (int s = 0; s < kMaxSplit; ++s)
    if (s < p.nsplit) {
      const float w = lv[s] * il;
#pragma unroll
      for (int bb = 0; bb < 4; ++bb)
#pragma unroll
        for (int r2 = 0; r2 < 2; ++r2)
#pragma unroll
          for (int e = 0; e < 8; ++e)
            acc[bb][8 * r2 + e] =
                fmaf(w, (float)pr[s % kPre][2 * bb + r2][e], acc[bb][8 * r2 + e]);
      if (s + kPre < p.nsplit) {
#pragma unroll
        for (int u = 0; u < 8; ++u)
          pr[s % kPre][u] = *(const bf16x8 *)(src + (s + kPre) * kPartialOBytes + u * 64 * 16);
      }
    }

  if (inter) {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    // (q W_q)^T = W_q^T q^T: rows = features, lane = query; four
    // independent chains, interleaved.
    f32x16 qp4[4];
#pragma unroll
    for (int bb = 0; bb < 4; ++bb) qp4[bb] = zero16();
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const int k0 = 16 * c + 8 * hl;
      bf16x8 wa[4];
#pragma unroll
      for (int bb = 0; bb < 4; ++bb) wa[bb] = tile_col_operand(Wt, k0, k0 + 4, lane, bb);
#pragma unroll
      for (int bb = 0; bb < 4; ++bb) qp4[bb] = mfma32(wa[bb], qop[c], qp4[bb]);
    }
    float ss = 0.f;
#pragma unroll
    for (int bb = 0; bb < 4; ++bb)
#pragma unroll
      for (int i = 0; i < 16; ++i) ss = fmaf(qp4[bb][i], qp4[bb][i], ss);
    ss += swap_halves(ss);
    const float inv = 1.f / fmaxf(sqrtf(ss), kL2Eps);
    // acc += O_inter^T = S^T Q'^T with Q' fed from the accumulators:
    // register 8*(g%2) + j of block g/2 holds feature 16g +
    // swap_bits23(8*(l/32) + j), i.e. rows 16g + 4*(l/32) + {0..3} and
    // 16g + 8 + 4*(l/32) + {0..3} of S.
#pragma unroll
    for (int g = 0; g < 8; ++g) {
      bf16x8 qb;
#pragma unroll
      for (int j = 0; j < 8; ++j) qb[j] = (bf16)(qp4[g >> 1][8 * (g & 1) + j] * inv);
      const int k0 = 16 * g + 4 * hl;
      bf16x8 sa[4];
#pragma unroll
      for (int bb = 0; bb < 4; ++bb) sa[bb] = tile_col_operand(St, k0, k0 + 8, lane, bb);
#pragma unroll
      for (int bb = 0; bb < 4; ++bb) acc[bb] = mfma32(sa[bb], qb, acc[bb]);
    }
  } else if (p.o_inter) {
    // A precomputed inter-frame term, in the accumulators' order: register
    // 4r + e of block bb is feature 32bb + 8r + 4(l/32) + e.
    const float *oi = p.o_inter + ((int64_t)b * p.L + qrow) * tok + (int64_t)h * D + 4 * hl;
#pragma unroll
    for (int bb = 0; bb < 4; ++bb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const f32x4 x = qrow < p.L ? *(const f32x4 *)(oi + 32 * bb + 8 * r) : zero4();
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[bb][4 * r + e] += x[e];
      }
  }

  // Output rows through LDS: the wave's 32 rows as a swizzled 32 x 256-byte
  // tile in Wt (free once every wave is past the inter-frame read), then
  // 16-byte units, 16 lanes per 256-byte row.
  __syncthreads();
  char *ot = Wt + wave * 32 * 256;
#pragma unroll
  for (int bb = 0; bb < 4; ++bb)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      bf16x4 t;
#pragma unroll
      for (int e = 0; e < 4; ++e) t[e] = (bf16)acc[bb][4 * r + e];
      *(bf16x4 *)(ot + tile_off(l32, 4 * bb + r) + 8 * hl) = t;
    }
  __builtin_amdgcn_s_waitcnt(0);
  __builtin_amdgcn_wave_barrier();
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int row = 4 * i + (lane >> 4), u = lane & 15;
    const int qr = qblk * kQBlock + wave * 32 + row;
    const bf16x8 t = *(const bf16x8 *)(ot + tile_off(row, u));
    if (qr < p.L) *(bf16x8 *)(p.out + ((int64_t)b * p.L + qr) * tok + (int64_t)h * D + 8 * u) = t;
  }
}

struct DeltaKParams {
  const bf16 *k, *v, *Wk, *Wv;
  const float *S, *beta;
  int H, L, nchunk, nitems;
  float *ws_dS;
};

// One chunk of 32*NT tokens (item = (stream, head, chunk), chunk fastest).
// bufA holds W_k, then K' (hi); bufB W_v, then K' (lo); 32 KB each.
template <int NT>
__device__ __forceinline__ void delta_body(const DeltaKParams p, int item, char *bufA, char *bufB,
                                           float *betas) {
  static_assert(NT >= 1 && NT <= 4, "token tiles per chunk");
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

  // (0) Weight tiles: wave w copies 4-row chunks 8w .. 8w+7 of each map;
  // lane (r4 = l/16, pos = l%16) fetches unit pos ^ swizzle of its row, so
  // the bytes land in the swizzled layout.
  {
    const bf16 *Wk = p.Wk + (int64_t)h * D * D;
    const bf16 *Wv = p.Wv + (int64_t)h * D * D;
    const int r4 = lane >> 4, pos = lane & 15;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int cc = 8 * wave + i, row = 4 * cc + r4;
      const int off = row * D + 8 * (pos ^ tile_swz(row & 15));
      global_to_lds16(Wk + off, bufA + cc * 1024);
      global_to_lds16(Wv + off, bufB + cc * 1024);
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
      for (int bb = 0; bb < 4; ++bb) wa[bb] = tile_col_operand(bufA, k0, k0 + 4, lane, bb);
#pragma unroll
      for (int bb = 0; bb < 4; ++bb) kt[bb] = mfma32(wa[bb], kop[c], kt[bb]);
    }
    float ss = 0.f;
#pragma unroll
    for (int bb = 0; bb < 4; ++bb)
#pragma unroll
      for (int i = 0; i < 16; ++i) ss = fmaf(kt[bb][i], kt[bb][i], ss);
    ss += swap_halves(ss);
    inv = 1.f / fmaxf(sqrtf(ss), kL2Eps);
  }
  // W_v[d_in][d_v] for this wave's columns as B operands (k = d_in).
  bf16x8 wv[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const int k0 = 16 * c + 8 * hl;
    wv[c] = tile_col_operand(bufB, k0, k0 + 4, lane, wave);
  }
  __syncthreads();  // every read of the weight tiles is done

  // K' rows (split bf16) over the weight tiles: row = token, column = d_k.
  if (wave < NT) {
    const int row = 32 * wave + l32;
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
        const int off = tile_off(row, 4 * bb + r) + 8 * hl;
        *(bf16x4 *)(bufA + off) = th;
        *(bf16x4 *)(bufB + off) = tl;
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
    f32x16 a0 = zero16(), a1 = zero16();
#pragma unroll
    for (int g = 0; g < 8; ++g) {
      const int off = tile_off(32 * tt + l32, 2 * g + hl);
      const bf16x8 ah = *(const bf16x8 *)(bufA + off);
      const bf16x8 al = *(const bf16x8 *)(bufB + off);
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
        ah[db] = tile_col_operand(bufA, k0, k0 + 8, lane, db);
        al[db] = tile_col_operand(bufB, k0, k0 + 8, lane, db);
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

struct TailKParams {
  CombineKParams c;
  DeltaKParams d;
  int delta_blocks;  // leading workgroups that run delta chunks (0: none)
  int per_xcd_d, per_xcd_c;
};

// Items of either kind are dealt so that each XCD gets a contiguous run
// (workgroups go to the 8 XCDs round-robin by linear id): the query blocks
// or chunks of one head share that XCD's L2 for the head's weights and
// state. Delta chunks take the first workgroup ids, so they start first.
__device__ __forceinline__ int xcd_item(int bid, int per_xcd) {
  return (bid & 7) * per_xcd + (bid >> 3);
}

template <int NT>
__global__ __launch_bounds__(256, 2) void tail_kernel(TailKParams P) {
  __shared__ __attribute__((aligned(1024))) char lds0[TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char lds1[TILE_BYTES];
  __shared__ float betas[32 * NT];
  const int bid = blockIdx.x;
  if (bid < P.delta_blocks) {
    const int item = xcd_item(bid, P.per_xcd_d);
    if (item < P.d.nitems) delta_body<NT>(P.d, item, lds0, lds1, betas);
  } else {
    const int item = xcd_item(bid - P.delta_blocks, P.per_xcd_c);
    if (item < P.c.nitems) combine_body(P.c, item, lds0, lds1);
  }
}

// S := alpha S + sum_c dS_c, one thread per 4 consecutive state values;
// the chunk partials are summed in chunk order, with up to 16 loads in
// flight per thread.
__global__ __launch_bounds__(64) void delta_apply_kernel(float *S, const float *alpha,
                                                         int arow4, const float *ws, int dd4,
                                                         int nchunk) {
  const int e = blockIdx.x * 64 + threadIdx.x;
  const int bh = blockIdx.y;
  if (e >= dd4) return;
  const f32x4 *w = (const f32x4 *)ws + (int64_t)bh * nchunk * dd4 + e;
  f32x4 *sp = (f32x4 *)S + (int64_t)bh * dd4 + e;
  const f32x4 sv = *sp;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int c0 = 0; c0 < nchunk; c0 += 16) {
    f32x4 t[16];
#pragma unroll
    for (int u = 0; u < 16; ++u)
      if (c0 + u < nchunk) t[u] = w[(int64_t)(c0 + u) * dd4];
#pragma unroll
    for (int u = 0; u < 16; ++u)
      if (c0 + u < nchunk) acc += t[u];
  }
  // Headwise: one gate per (stream, head) (arow4 = 0). Elementwise: one gate
  // per d_k row; a row holds arow4 groups of 4 values.
  const float a = arow4 ? alpha[(int64_t)bh * (dd4 / arow4) + e / arow4] : alpha[bh];
  f32x4 r;
#pragma unroll
  for (int u = 0; u < 4; ++u) r[u] = fmaf(a, sv[u], acc[u]);
  *sp = r;
}

__global__ __launch_bounds__(256) void fill_state_kernel(float *dst, const float *src, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) dst[i] = src ? src[i] : 0.f;
}

}  // namespace

int delta_chunk_tokens(int64_t B, int64_t H, int64_t L) {
  const int64_t items = B * H * ((L + 95) / 96 + (L + kQBlock - 1) / kQBlock);
  return items <= 512 ? 96 : 128;
}

hipError_t launch_tail_bf16(const CombineArgs &c, const DeltaArgs *d, hipStream_t s) {
  if (d && d->chunk != 96 && d->chunk != 128) return hipErrorInvalidValue;
  TailKParams P;
  P.c.ws_o = (const char *)c.ws_o;
  P.c.ws_ml = c.ws_ml;
  P.c.q = (const bf16 *)c.q;
  P.c.Wq = (const bf16 *)c.Wq;
  P.c.S = c.S;
  P.c.H = c.H;
  P.c.L = c.L;
  P.c.nqblk = c.plan.nqblk;
  P.c.nsplit = c.plan.nsplit;
  P.c.nitems = c.B * c.H * c.plan.nqblk;
  P.c.out = (bf16 *)c.out;
  P.c.o_inter = c.Wq ? nullptr : c.o_inter;
  P.per_xcd_c = (P.c.nitems + 7) / 8;
  P.d = DeltaKParams{};
  P.delta_blocks = 0;
  P.per_xcd_d = 0;
  if (d) {
    P.d.k = (const bf16 *)d->k;
    P.d.v = (const bf16 *)d->v;
    P.d.Wk = (const bf16 *)d->Wk;
    P.d.Wv = (const bf16 *)d->Wv;
    P.d.S = d->S;
    P.d.beta = d->beta;
    P.d.H = d->H;
    P.d.L = d->L;
    P.d.nchunk = d->nchunk;
    P.d.nitems = d->B * d->H * d->nchunk;
    P.d.ws_dS = d->ws_dS;
    P.per_xcd_d = (P.d.nitems + 7) / 8;
    P.delta_blocks = 8 * P.per_xcd_d;
  }
  const unsigned blocks = (unsigned)(P.delta_blocks + 8 * P.per_xcd_c);
  if (d && d->chunk == 96)
    hipLaunchKernelGGL(tail_kernel<3>, dim3(blocks), dim3(256), 0, s, P);
  else
    hipLaunchKernelGGL(tail_kernel<4>, dim3(blocks), dim3(256), 0, s, P);
  return hipGetLastError();
}

hipError_t launch_delta_apply(float *S, const float *alpha, bool elementwise, const float *ws_dS,
                              int B, int H, int d, int nchunk, hipStream_t s) {
  const int dd4 = d * d / 4;
  dim3 grid((unsigned)((dd4 + 63) / 64), (unsigned)(B * H));
  hipLaunchKernelGGL(delta_apply_kernel, grid, dim3(64), 0, s, S, alpha, elementwise ? d / 4 : 0,
                     ws_dS, dd4, nchunk);
  return hipGetLastError();
}

hipError_t launch_fill_state(float *dst, const float *src, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  dim3 grid((unsigned)((n + 255) / 256));
  hipLaunchKernelGGL(fill_state_kernel, grid, dim3(256), 0, s, dst, src, n);
  return hipGetLastError();
}

}  // namespace arl2
