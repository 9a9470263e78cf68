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
#include "mfma_stage.h"

#include <math.h>

namespace arl2 {
namespace {

constexpr int D = 128;
constexpr int KB = kKeyTile;  // 64 keys per LDS tile
constexpr int KS_LD = D + 8;  // K tile row stride (bf16): 272 B, conflict-free b128 reads
constexpr int VT_LD = KB + 8; // V^T tile row stride (bf16): 144 B

struct AttnKParams {
  const bf16 *q, *k, *v;
  int H, Lq, Lk, nsplit, kps, nqblk;
  float *ws_o, *ws_ml;
  float scale;  // log2(e) / sqrt(d)
};

__global__ __launch_bounds__(256) void attn_partial_kernel(AttnKParams p) {
  __shared__ __attribute__((aligned(16))) bf16 Ks[KB * KS_LD];
  __shared__ __attribute__((aligned(16))) bf16 Vt[D * VT_LD];

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, hl = lane >> 5, l32 = lane & 31;
  const int split = blockIdx.x % p.nsplit;
  const int qblk = blockIdx.x / p.nsplit;
  const int h = blockIdx.y, b = blockIdx.z;
  const int64_t tok = (int64_t)p.H * D;
  const bf16 *qbase = p.q + ((int64_t)b * p.Lq * p.H + h) * D;
  const bf16 *kbase = p.k + ((int64_t)b * p.Lk * p.H + h) * D;
  const bf16 *vbase = p.v + ((int64_t)b * p.Lk * p.H + h) * D;

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

  const int kbeg = split * p.kps;
  const int kend = min(p.Lk, kbeg + p.kps);

  // Tile staging: K as 4 rows x 16 B per thread (coalesced rows), V as
  // 4 consecutive keys x 8 head-dim values per thread (for the transpose).
  const int kd = tid & 15, kr0 = tid >> 4;
  const int vg = tid & 15, vd = tid >> 4;
  const int vpos = 4 * swap_bits01(vg);
  bf16x8 kreg[4], vreg[4];

  auto load_tile = [&](int t0) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int key = t0 + kr0 + 16 * r;
      kreg[r] = key < kend ? *(const bf16x8 *)(kbase + key * tok + 8 * kd) : zero_bf16x8();
      const int vkey = t0 + 4 * vg + r;
      vreg[r] = vkey < kend ? *(const bf16x8 *)(vbase + vkey * tok + 8 * vd) : zero_bf16x8();
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int r = 0; r < 4; ++r) *(bf16x8 *)(Ks + (kr0 + 16 * r) * KS_LD + 8 * kd) = kreg[r];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      bf16x4 t;
      t[0] = vreg[0][e];
      t[1] = vreg[1][e];
      t[2] = vreg[2][e];
      t[3] = vreg[3][e];
      *(bf16x4 *)(Vt + (8 * vd + e) * VT_LD + vpos) = t;
    }
  };

  load_tile(kbeg);
  for (int t0 = kbeg; t0 < kend; t0 += KB) {
    __syncthreads();  // every wave is done reading the previous tile
    store_tile();
    __syncthreads();
    if (t0 + KB < kend) load_tile(t0 + KB);
    const int nvalid = kend - t0;

    // S^T for two 32-key sub-blocks: rows = keys, columns = this wave's queries.
    f32x16 s[2];
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
      s[sb] = zero16();
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const bf16x8 a = *(const bf16x8 *)(Ks + (32 * sb + l32) * KS_LD + 16 * c + 8 * hl);
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

    // Online softmax in the log2 domain (every tile has a valid key, so the
    // new maximum is finite).
    float mx = -INFINITY;
#pragma unroll
    for (int sb = 0; sb < 2; ++sb)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[sb][i]);
    mx = fmaxf(mx, swap_halves(mx));
    const float mnew = fmaxf(m, mx * p.scale);
    if (wave_any(mnew != m)) {
      const float r = exp2_fast(m - mnew);
#pragma unroll
      for (int bb = 0; bb < 4; ++bb)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[bb][i] *= r;
      lsum *= r;
    }
    m = mnew;

    bf16x8 pb[4];
    float ps = 0.f;
#pragma unroll
    for (int sb = 0; sb < 2; ++sb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float pv = exp2_fast(fmaf(s[sb][i], p.scale, -mnew));
        ps += pv;
        pb[2 * sb + (i >> 3)][i & 7] = (bf16)pv;
      }
    lsum += ps;

    // O^T += V^T P^T over the tile's 64 keys (4 steps of 16).
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
#pragma unroll
      for (int bb = 0; bb < 4; ++bb) {
        const bf16x8 a = *(const bf16x8 *)(Vt + (32 * bb + l32) * VT_LD + 16 * kk + 8 * hl);
        o[bb] = mfma32(a, pb[kk], o[bb]);
      }
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

__global__ __launch_bounds__(256) void inter_combine_kernel(CombineKParams p) {
  __shared__ __attribute__((aligned(16))) bf16 WqT[D * W_LD];
  __shared__ __attribute__((aligned(16))) bf16 ST[D * W_LD];

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, hl = lane >> 5, l32 = lane & 31;
  const int qblk = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int64_t tok = (int64_t)p.H * D;
  const int qrow = qblk * kQBlock + wave * 32 + l32;

  f32x16 oi[4];  // O_inter^T: lane = query, registers = d_v
#pragma unroll
  for (int bb = 0; bb < 4; ++bb) oi[bb] = zero16();

  if (p.with_inter) {
    stage_weight_T(p.Wq + (int64_t)h * D * D, WqT, tid);
    stage_state_T(p.S + ((int64_t)b * p.H + h) * D * D, ST, nullptr, tid);
    __syncthreads();

    bf16x8 qop[8];
    if (qrow < p.L) {
      const bf16 *qp = p.q + ((int64_t)b * p.L * p.H + h) * D + qrow * tok + 8 * hl;
#pragma unroll
      for (int c = 0; c < 8; ++c) qop[c] = *(const bf16x8 *)(qp + 16 * c);
    } else {
#pragma unroll
      for (int c = 0; c < 8; ++c) qop[c] = zero_bf16x8();
    }
    // (q W_q)^T = W_q^T q^T: lane = query, registers = output features.
    f32x16 qp4[4];
#pragma unroll
    for (int bb = 0; bb < 4; ++bb) {
      qp4[bb] = zero16();
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const bf16x8 a = *(const bf16x8 *)(WqT + (32 * bb + l32) * W_LD + 16 * c + 8 * hl);
        qp4[bb] = mfma32(a, qop[c], qp4[bb]);
      }
    }
    float ss = 0.f;
#pragma unroll
    for (int bb = 0; bb < 4; ++bb)
#pragma unroll
      for (int i = 0; i < 16; ++i) ss = fmaf(qp4[bb][i], qp4[bb][i], ss);
    ss += swap_halves(ss);
    const float inv = 1.f / fmaxf(sqrtf(ss), kL2Eps);
    // O_inter^T = S^T Q'^T with Q' fed straight from the accumulators.
#pragma unroll
    for (int g = 0; g < 8; ++g) {
      bf16x8 qb;
#pragma unroll
      for (int j = 0; j < 8; ++j) qb[j] = (bf16)(qp4[g >> 1][8 * (g & 1) + j] * inv);
#pragma unroll
      for (int bb = 0; bb < 4; ++bb) {
        const bf16x8 a = *(const bf16x8 *)(ST + (32 * bb + l32) * W_LD + 16 * g + 8 * hl);
        oi[bb] = mfma32(a, qb, oi[bb]);
      }
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
  // Enough workgroups to cover the 256 compute units about twice, without
  // splitting a key range below two tiles.
  int64_t ns = (448 + base - 1) / base;
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
  dim3 grid((unsigned)(a.plan.nqblk * a.plan.nsplit), (unsigned)a.H, (unsigned)a.B);
  hipLaunchKernelGGL(attn_partial_kernel, grid, dim3(256), 0, s, p);
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
