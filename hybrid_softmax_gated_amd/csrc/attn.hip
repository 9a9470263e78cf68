// Intra-frame softmax attention (bf16, d = 128) on the gfx950 matrix cores,
// and the epilogue that merges its key-range partials, adds the inter-frame
// read O_inter = Q' S and writes the layer output.
//
// Method: "Technical Summary: Attend Locally, Remember Linearly (ARL2)",
// section 2.1 — the intra-frame branch keeps full bidirectional softmax
// attention inside the frame; the inter-frame branch reads the fixed-size
// state with feature-mapped, L2-normalised queries; every token of the frame
// reads the same pre-update state (section 2.2, frame-level access).
//
// Data layout in HBM: q, k, v, out are token-major [B][L][H][128] bf16, so a
// head's row of 128 values is 256 contiguous bytes and consecutive tokens of
// one head are H*256 bytes apart.
//
// Attention kernel (one workgroup = 4 wavefronts = 128 queries of one head,
// one contiguous key range):
//  * each wavefront keeps its 32 queries in registers as MFMA B operands and
//    computes the transposed score tile S^T = K Q^T (keys on rows), so every
//    lane owns one query: the row max and row sum of the online softmax are
//    in-register reductions plus one exchange between the wave halves;
//  * K tiles are staged in LDS row-major, V tiles transposed (head dim on
//    rows) with keys in the swap_bits23 order, so that the softmax
//    probabilities leave the score accumulators and enter O^T = V^T P^T as
//    the B operand without any data movement;
//  * the next tile's global loads are issued before the current tile's
//    MFMAs (register double buffering);
//  * the unnormalised O^T, the row max (log2 domain) and the row sum are
//    written per key range; the epilogue merges the ranges.
#include "arl2_device.h"
#include "arl2_kernels.h"

#include <math.h>

namespace arl2 {
namespace {

constexpr int D = 128;
constexpr int KB = kKeyTile;  // 64 keys per LDS tile

struct AttnKParams {
  const bf16 *q, *k, *v;
  int H, Lq, Lk, nsplit, kps, nqblk;
  int nitems, per_xcd;  // work items and items per XCD (see item_of)
  float *ws_o, *ws_ml;
  float scale;  // log2(e) / sqrt(d)
};

// Work items are (stream, head, split, query block) with the query block
// fastest, so that consecutive items share one key range of one head.
// Workgroups are dealt to the 8 XCDs round-robin by linear id; item_of gives
// every XCD a contiguous run of items, so the K/V rows a run touches stay in
// that XCD's L2.
__device__ __forceinline__ int item_of(int bid, int per_xcd) {
  return (bid & 7) * per_xcd + (bid >> 3);
}

// Issue the direct global->LDS copy of one 64-key tile (64 rows of 256 B,
// swizzled): 16 chunks of 4 rows, 4 per wavefront. Rows past the key range
// re-read the last valid row (finite values; their scores are masked).
__device__ __forceinline__ void issue_tile(const bf16 *__restrict__ base, int64_t tok, int t0,
                                           int kend, bf16 *tile, int wave, int lane) {
  const int r4 = lane >> 4, pos = lane & 15;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int cc = 4 * wave + i;
    const int row = 4 * cc + r4;
    const int key = min(t0 + row, kend - 1);
    const int unit = pos ^ tile_swz(row & 15);
    global_to_lds16(base + key * tok + 8 * unit, tile + cc * 512);
  }
}

// Register-staged copy of one 64-key tile into the same swizzled layout:
// thread t owns rows t/16 + 16i (i = 0..3), unit t%16.
__device__ __forceinline__ void load_tile_regs(const bf16 *__restrict__ base, int64_t tok, int t0,
                                               int kend, int tid, bf16x8 (&r)[4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int key = min(t0 + (tid >> 4) + 16 * i, kend - 1);
    r[i] = *(const bf16x8 *)(base + key * tok + 8 * (tid & 15));
  }
}
__device__ __forceinline__ void store_tile_regs(char *tile, int tid, const bf16x8 (&r)[4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
    *(bf16x8 *)(tile + tile_off((tid >> 4) + 16 * i, tid & 15)) = r[i];
}

__global__ __launch_bounds__(256, 2) void attn_partial_kernel(AttnKParams p) {
  __shared__ __attribute__((aligned(1024))) bf16 Kt0[KB * D];
  __shared__ __attribute__((aligned(1024))) bf16 Kt1[KB * D];
  __shared__ __attribute__((aligned(1024))) bf16 Vt0[KB * D];
  __shared__ __attribute__((aligned(1024))) bf16 Vt1[KB * D];

  const int item = item_of(blockIdx.x, p.per_xcd);
  if (item >= p.nitems) return;
  const int qblk = item % p.nqblk;
  int rest = item / p.nqblk;
  const int split = rest % p.nsplit;
  rest /= p.nsplit;
  const int h = rest % p.H, b = rest / p.H;

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, hl = lane >> 5, l32 = lane & 31;
  const int64_t tok = (int64_t)p.H * D;
  const bf16 *qbase = p.q + ((int64_t)b * p.Lq * p.H + h) * D;
  const bf16 *kbase = p.k + ((int64_t)b * p.Lk * p.H + h) * D;
  const bf16 *vbase = p.v + ((int64_t)b * p.Lk * p.H + h) * D;
  const int kbeg = split * p.kps;
  const int kend = min(p.Lk, kbeg + p.kps);

  bf16x8 kreg[4], vreg[4];
  load_tile_regs(kbase, tok, kbeg, kend, tid, kreg);
  load_tile_regs(vbase, tok, kbeg, kend, tid, vreg);
  store_tile_regs((char *)Kt0, tid, kreg);
  store_tile_regs((char *)Vt0, tid, vreg);

  // The wavefront's 32 queries as B operands: lane l holds query l%32,
  // head-dim elements 16c + 8*(l/32) .. +7.
  const int qrow = qblk * kQBlock + wave * 32 + l32;
  bf16x8 qop[8];
  if (qrow < p.Lq) {
    const bf16 *qp = qbase + qrow * tok + 8 * hl;
#pragma unroll
    for (int c = 0; c < 8; ++c) qop[c] = *(const bf16x8 *)(qp + 16 * c);
  } else {
#pragma unroll
    for (int c = 0; c < 8; ++c) qop[c] = zero_bf16x8();
  }

  f32x16 o[4];
#pragma unroll
  for (int bb = 0; bb < 4; ++bb) o[bb] = zero16();
  float m = -INFINITY, lsum = 0.f;

  // Per-lane LDS byte offsets. K (A operand of S^T = K Q^T): row l%32 of a
  // 32-key sub-block, unit 2c + l/32. V (A operand of O^T = V^T P^T, read
  // transposed): lane i of group g reads row 8r + 4*(g/2) + i/4 (r = 0, 1)
  // of a 16-key step, columns 32bb + 16*(g%2) + 4*(i%4) .. +3.
  int koff[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) koff[c] = tile_off(l32, 2 * c + hl);
  const int gi = lane & 15, g = lane >> 4;
  int voff[2][4];
#pragma unroll
  for (int r = 0; r < 2; ++r)
#pragma unroll
    for (int bb = 0; bb < 4; ++bb) {
      const int row = 8 * r + 4 * (g >> 1) + (gi >> 2);
      const int col = 32 * bb + 16 * (g & 1) + 4 * (gi & 3);
      voff[r][bb] = tile_off(row, col >> 3) + 2 * (col & 7);
    }

  __builtin_amdgcn_s_waitcnt(0);  // Q operands and the first tile have landed
  __syncthreads();

  int buf = 0;
  for (int t0 = kbeg; t0 < kend; t0 += KB) {
    const char *Kc = (const char *)(buf ? Kt1 : Kt0);
    const char *Vc = (const char *)(buf ? Vt1 : Vt0);
    const bool more = t0 + KB < kend;
    if (more) {
      load_tile_regs(kbase, tok, t0 + KB, kend, tid, kreg);
      load_tile_regs(vbase, tok, t0 + KB, kend, tid, vreg);
    }
    const int nvalid = kend - t0;

    // S^T for two 32-key sub-blocks: rows = keys, columns = this wave's queries.
    f32x16 s[2];
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
      s[sb] = zero16();
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const bf16x8 a = *(const bf16x8 *)(Kc + sb * 32 * 256 + koff[c]);
        s[sb] = mfma32(a, qop[c], s[sb]);
      }
    }
    if (nvalid < KB) {
#pragma unroll
      for (int sb = 0; sb < 2; ++sb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = 32 * sb + 8 * (i >> 2) + 4 * hl + (i & 3);
          if (key >= nvalid) s[sb][i] = -INFINITY;
        }
    }

    // Online softmax in the log2 domain. The running maximum is only moved
    // when a new score exceeds it by more than 2^8; in between, exponents
    // stay below 2^8, which fp32 sums and bf16 probabilities carry exactly
    // as well as values below 1 (every tile has a valid key, so the first
    // tile always sets a finite maximum).
    float mx = -INFINITY;
#pragma unroll
    for (int sb = 0; sb < 2; ++sb)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[sb][i]);
    mx = fmaxf(mx, swap_halves(mx)) * p.scale;
    if (wave_any(mx > m + 8.f)) {
      const float mnew = fmaxf(m, mx);
      const float r = exp2_fast(m - mnew);
#pragma unroll
      for (int bb = 0; bb < 4; ++bb)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[bb][i] *= r;
      lsum *= r;
      m = mnew;
    }

    bf16x8 pb[4];
    float ps = 0.f;
#pragma unroll
    for (int sb = 0; sb < 2; ++sb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float pv = exp2_fast(fmaf(s[sb][i], p.scale, -m));
        ps += pv;
        pb[2 * sb + (i >> 3)][i & 7] = (bf16)pv;
      }
    lsum += ps;

    // O^T += V^T P^T over the tile's 64 keys (4 steps of 16).
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
#pragma unroll
      for (int bb = 0; bb < 4; ++bb) {
        const s16x4 lo = lds_read_tr16(Vc + kk * 16 * 256 + voff[0][bb]);
        const s16x4 hi = lds_read_tr16(Vc + kk * 16 * 256 + voff[1][bb]);
        const bf16x8 a = __builtin_bit_cast(
            bf16x8, (short __attribute__((ext_vector_type(8)))){lo[0], lo[1], lo[2], lo[3], hi[0],
                                                                hi[1], hi[2], hi[3]});
        o[bb] = mfma32(a, pb[kk], o[bb]);
      }

    if (more) {
      store_tile_regs((char *)(buf ? Kt0 : Kt1), tid, kreg);
      store_tile_regs((char *)(buf ? Vt0 : Vt1), tid, vreg);
    }
    __syncthreads();  // the next tile is in LDS and nobody reads this one any more
    buf ^= 1;
  }

  const int64_t blk = (((int64_t)b * p.H + h) * p.nqblk + qblk) * p.nsplit + split;
  float *wo = p.ws_o + blk * kPartialO + wave * 64 * 64;
#pragma unroll
  for (int bb = 0; bb < 4; ++bb)
#pragma unroll
    for (int i = 0; i < 16; ++i) wo[(16 * bb + i) * 64 + lane] = o[bb][i];
  const float lt = lsum + swap_halves(lsum);
  float *wml = p.ws_ml + blk * kPartialML + wave * 64;
  if (hl == 0) {
    wml[l32] = m;
    wml[32 + l32] = lt;
  }
}

struct CombineKParams {
  const bf16 *q, *Wq;
  const float *S;
  int H, L, nqblk, nsplit;
  const float *ws_o, *ws_ml;
  bf16 *out;
  int with_inter;
};

// A operand (rows = 32 columns 32bb .. 32bb+31 of the tile, k = 8 tile
// rows) read transposed from a swizzled row-major 128x128 bf16 tile: rows
// k0 .. k0+3 land in elements 0..3 and rows k1 .. k1+3 in elements 4..7.
__device__ __forceinline__ bf16x8 tile_col_operand(const char *tile, int k0, int k1, int lane,
                                                   int bb) {
  const int gi = lane & 15, g = lane >> 4;
  const int col = 32 * bb + 16 * (g & 1) + 4 * (gi & 3);
  const s16x4 lo = lds_read_tr16(tile + tile_off(k0 + (gi >> 2), col >> 3) + 2 * (col & 7));
  const s16x4 hi = lds_read_tr16(tile + tile_off(k1 + (gi >> 2), col >> 3) + 2 * (col & 7));
  return __builtin_bit_cast(bf16x8, (short __attribute__((ext_vector_type(8)))){
                                        lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
}

__global__ __launch_bounds__(256) void inter_combine_kernel(CombineKParams p) {
  __shared__ __attribute__((aligned(1024))) bf16 Wt[D * D];   // W_q[h], row-major [din][dout]
  __shared__ __attribute__((aligned(1024))) bf16 St[D * D];   // bf16(S[b][h]), row-major [dk][dv]

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, hl = lane >> 5, l32 = lane & 31;
  const int qblk = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int64_t tok = (int64_t)p.H * D;
  const int qrow = qblk * kQBlock + wave * 32 + l32;

  f32x16 oi[4];  // O_inter^T: lane = query, registers = d_v
#pragma unroll
  for (int bb = 0; bb < 4; ++bb) oi[bb] = zero16();

  if (p.with_inter) {
    // W_q[h]: 32 chunks of 4 rows, copied straight into LDS (8 per wave).
    const bf16 *W = p.Wq + (int64_t)h * D * D;
    const int r4 = lane >> 4, pos = lane & 15;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int cc = 8 * wave + i, row = 4 * cc + r4;
      global_to_lds16(W + row * D + 8 * (pos ^ tile_swz(row & 15)), Wt + cc * 512);
    }
    // S[b][h] rounded to bf16: thread t converts rows t/16 + 16i, unit t%16.
    const float *Sh = p.S + ((int64_t)b * p.H + h) * D * D;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int row = (tid >> 4) + 16 * i, u = tid & 15;
      const f32x4 a = *(const f32x4 *)(Sh + row * D + 8 * u);
      const f32x4 c = *(const f32x4 *)(Sh + row * D + 8 * u + 4);
      bf16x8 t;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        t[e] = (bf16)a[e];
        t[4 + e] = (bf16)c[e];
      }
      *(bf16x8 *)((char *)St + tile_off(row, u)) = t;
    }
    bf16x8 qop[8];
    if (qrow < p.L) {
      const bf16 *qp = p.q + ((int64_t)b * p.L * p.H + h) * D + qrow * tok + 8 * hl;
#pragma unroll
      for (int c = 0; c < 8; ++c) qop[c] = *(const bf16x8 *)(qp + 16 * c);
    } else {
#pragma unroll
      for (int c = 0; c < 8; ++c) qop[c] = zero_bf16x8();
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    // (q W_q)^T = W_q^T q^T: lane = query, registers = output features.
    f32x16 qp4[4];
#pragma unroll
    for (int bb = 0; bb < 4; ++bb) {
      qp4[bb] = zero16();
#pragma unroll
      for (int c = 0; c < 8; ++c)
        qp4[bb] = mfma32(tile_col_operand((const char *)Wt, 16 * c + 8 * hl, 16 * c + 8 * hl + 4,
                                          lane, bb),
                         qop[c], qp4[bb]);
    }
    float ss = 0.f;
#pragma unroll
    for (int bb = 0; bb < 4; ++bb)
#pragma unroll
      for (int i = 0; i < 16; ++i) ss = fmaf(qp4[bb][i], qp4[bb][i], ss);
    ss += swap_halves(ss);
    const float inv = 1.f / fmaxf(sqrtf(ss), kL2Eps);
    // O_inter^T = S^T Q'^T, Q' fed straight from the accumulators: register
    // 8*(g%2) + j of block g/2 holds feature 16g + swap_bits23(8*(l/32) + j),
    // i.e. rows 16g + 4*(l/32) + {0..3} and 16g + 8 + 4*(l/32) + {0..3}.
#pragma unroll
    for (int g = 0; g < 8; ++g) {
      bf16x8 qb;
#pragma unroll
      for (int j = 0; j < 8; ++j) qb[j] = (bf16)(qp4[g >> 1][8 * (g & 1) + j] * inv);
#pragma unroll
      for (int bb = 0; bb < 4; ++bb)
        oi[bb] = mfma32(
            tile_col_operand((const char *)St, 16 * g + 4 * hl, 16 * g + 8 + 4 * hl, lane, bb), qb,
            oi[bb]);
    }
  }

  // Merge the key-range partials of the intra-frame branch.
  const int64_t blk0 = (((int64_t)b * p.H + h) * p.nqblk + qblk) * p.nsplit;
  float M = -INFINITY;
  for (int s = 0; s < p.nsplit; ++s)
    M = fmaxf(M, p.ws_ml[(blk0 + s) * kPartialML + wave * 64 + l32]);
  f32x16 o[4];
#pragma unroll
  for (int bb = 0; bb < 4; ++bb) o[bb] = zero16();
  float Lt = 0.f;
  for (int s = 0; s < p.nsplit; ++s) {
    const float *ml = p.ws_ml + (blk0 + s) * kPartialML + wave * 64;
    const float w = exp2_fast(ml[l32] - M);
    Lt = fmaf(w, ml[32 + l32], Lt);
    const float *po = p.ws_o + (blk0 + s) * kPartialO + wave * 64 * 64 + lane;
#pragma unroll
    for (int bb = 0; bb < 4; ++bb)
#pragma unroll
      for (int i = 0; i < 16; ++i) o[bb][i] = fmaf(w, po[(16 * bb + i) * 64], o[bb][i]);
  }
  const float invl = 1.f / Lt;

  if (qrow < p.L) {
    bf16 *op = p.out + ((int64_t)b * p.L * p.H + h) * D + qrow * tok;
#pragma unroll
    for (int bb = 0; bb < 4; ++bb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        bf16x4 t;
#pragma unroll
        for (int e = 0; e < 4; ++e) t[e] = (bf16)fmaf(o[bb][4 * r + e], invl, oi[bb][4 * r + e]);
        *(bf16x4 *)(op + 32 * bb + 8 * r + 4 * hl) = t;
      }
  }
}

}  // namespace

AttnPlan plan_attention(int64_t B, int64_t H, int64_t Lq, int64_t Lk) {
  AttnPlan pl;
  pl.nqblk = (int)((Lq + kQBlock - 1) / kQBlock);
  const int64_t base = B * H * pl.nqblk;
  // Two workgroups fit on a compute unit: aim for at most 2 x 256 work
  // items, without splitting a key range below two tiles.
  int64_t ns = 512 / base;
  const int64_t max_by_keys = (Lk + 2 * kKeyTile - 1) / (2 * kKeyTile);
  if (ns > max_by_keys) ns = max_by_keys;
  if (ns > 16) ns = 16;
  if (ns < 1) ns = 1;
  int64_t kps = (Lk + ns - 1) / ns;
  kps = (kps + kKeyTile - 1) / kKeyTile * kKeyTile;
  pl.keys_per_split = (int)kps;
  pl.nsplit = (int)((Lk + kps - 1) / kps);  // every split holds at least one key
  return pl;
}

hipError_t launch_attn_partial_bf16(const AttnArgs &a, hipStream_t s) {
  AttnKParams p;
  p.q = (const bf16 *)a.q;
  p.k = (const bf16 *)a.k;
  p.v = (const bf16 *)a.v;
  p.H = a.H;
  p.Lq = a.Lq;
  p.Lk = a.Lk;
  p.nsplit = a.plan.nsplit;
  p.kps = a.plan.keys_per_split;
  p.nqblk = a.plan.nqblk;
  p.ws_o = a.ws_o;
  p.ws_ml = a.ws_ml;
  p.scale = kLog2e / sqrtf((float)D);
  p.nitems = a.B * a.H * a.plan.nsplit * a.plan.nqblk;
  p.per_xcd = (p.nitems + 7) / 8;
  hipLaunchKernelGGL(attn_partial_kernel, dim3((unsigned)(8 * p.per_xcd)), dim3(256), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_inter_combine_bf16(const CombineArgs &a, hipStream_t s) {
  CombineKParams p;
  p.q = (const bf16 *)a.q;
  p.Wq = (const bf16 *)a.Wq;
  p.S = a.S;
  p.H = a.H;
  p.L = a.L;
  p.nqblk = a.plan.nqblk;
  p.nsplit = a.plan.nsplit;
  p.ws_o = a.ws_o;
  p.ws_ml = a.ws_ml;
  p.out = (bf16 *)a.out;
  p.with_inter = a.with_inter ? 1 : 0;
  dim3 grid((unsigned)a.plan.nqblk, (unsigned)a.H, (unsigned)a.B);
  hipLaunchKernelGGL(inter_combine_kernel, grid, dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace arl2
