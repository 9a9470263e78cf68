// Intra-frame softmax attention (bf16, d = 128) on the gfx950 matrix cores,
// and the combine kernel that merges its key-range partials with the
// inter-frame read O_inter = Q' S and writes the layer output.
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
// one contiguous key range; two workgroups per compute unit):
//  * each wavefront keeps its 32 queries in registers as MFMA B operands and
//    computes the transposed score tile S^T = K Q^T (keys on rows), so every
//    lane owns one query: the row max and row sum of the online softmax are
//    in-register reductions plus one exchange between the wave halves;
//  * K and V tiles of 64 keys are staged in LDS row-major with a 16-byte
//    XOR swizzle (no bank conflicts for either read pattern); V is read as
//    the A operand of O^T = V^T P^T with the LDS transpose read, in the key
//    order that lets the softmax probabilities leave the score accumulators
//    and enter the next MFMA as its B operand with no data movement;
//  * double-buffered tiles: the next tile's buffer loads are issued before
//    the current tile's MFMAs and written to LDS after them (one barrier per
//    tile); the loop is unrolled by two so every LDS address is a constant
//    offset from a per-lane register;
//  * per key range it writes O/l in bf16, in the accumulators' register
//    order (16-byte coalesced stores), and the row max (log2 domain) and row
//    sum in fp32.
//
// Combine kernel (one workgroup = 128 queries of one head): the inter-frame
// read (q W_q, L2 norms, Q' S on the matrix cores, with W_q and bf16(S) in
// LDS), the merge of the key ranges in fp32, the sum of the two branches,
// and the bf16 output rows, transposed through LDS into 256-byte stores.
#include "arl2_device.h"
#include "arl2_kernels.h"

#include <math.h>

#include <type_traits>

namespace arl2 {
namespace {

constexpr int D = 128;
constexpr int KB = kKeyTile;         // 64 keys per LDS tile
constexpr int TILE_BYTES = KB * D * 2;  // 16 KB

struct AttnKParams {
  const bf16 *q, *k, *v;
  int H, Lq, Lk, nsplit, kps0, kps, nqblk;
  int nitems, per_xcd;  // work items and items per XCD (see item_of)
  char *ws_o;           // O/l partials, kPartialOBytes per block
  float *ws_ml;         // (max, sum) per query, kPartialML floats per block
  float scale;          // log2(e) / sqrt(d)
};

// Work items are (stream, head, split, query block) with the query block
// fastest, so that consecutive items share one key range of one head.
// Workgroups are dealt to the 8 XCDs round-robin by linear id; item_of gives
// every XCD a contiguous run of items, so the K/V rows a run touches stay in
// that XCD's L2.
__device__ __forceinline__ int item_of(int bid, int per_xcd) {
  return (bid & 7) * per_xcd + (bid >> 3);
}

__global__ __launch_bounds__(256, 2) void attn_partial_kernel(AttnKParams p) {
  // Double-buffered K and V tiles, each its own array so that the compiler
  // sees the copies into one buffer and the reads of the other as disjoint.
  __shared__ __attribute__((aligned(1024))) char Ks0[TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char Ks1[TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char Vs0[TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char Vs1[TILE_BYTES];

  const int item = item_of(blockIdx.x, p.per_xcd);
  if (item >= p.nitems) return;
  const int qblk = item % p.nqblk;
  int rest = item / p.nqblk;
  const int split = rest % p.nsplit;
  rest /= p.nsplit;
  const int h = rest % p.H, b = rest / p.H;

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, hl = lane >> 5, l32 = lane & 31;
  const int64_t tok = (int64_t)p.H * D;     // elements between tokens
  const int64_t tokB = tok * 2;             // bytes between tokens
  const bf16 *qbase = p.q + ((int64_t)b * p.Lq * p.H + h) * D;
  const char *kbase = (const char *)(p.k + ((int64_t)b * p.Lk * p.H + h) * D);
  const char *vbase = (const char *)(p.v + ((int64_t)b * p.Lk * p.H + h) * D);
  const int kbeg = split == 0 ? 0 : p.kps0 + (split - 1) * p.kps;
  const int kend = min(p.Lk, split == 0 ? p.kps0 : kbeg + p.kps);

  // Tile copies: wavefront w copies chunks 4w .. 4w+3 of 4 rows (1 KB) each;
  // lane (r4 = l/16, pos = l%16) of chunk cc fetches row 4cc + r4, 16-byte
  // unit pos ^ swizzle, so the bytes land in the swizzled layout.
  int doff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = 4 * (4 * wave + i) + (lane >> 4);
    doff[i] = (int)(row * tokB) + 16 * ((lane & 15) ^ tile_swz(row & 15));
  }
  // Copy the tile starting at key t0 into (kt, vt); rows at or past kend
  // read as zeros.
  auto copy_tile = [&](int t0, char *kt, char *vt) {
    const int64_t span = (int64_t)(kend - t0) * tokB;
    const uint32_t n = (uint32_t)(span < (int64_t)0x7fffffff ? span : (int64_t)0x7fffffff);
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(kbase + t0 * tokB, n);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(vbase + t0 * tokB, n);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      buffer_to_lds16(rk, kt + (4 * wave + i) * 1024, doff[i]);
      buffer_to_lds16(rv, vt + (4 * wave + i) * 1024, doff[i]);
    }
  };

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

  copy_tile(kbeg, Ks0, Vs0);

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

  // One 64-key tile from buffer BUF; the next tile is copied into the other
  // buffer meanwhile. Returns false after the last tile.
  auto step = [&](auto bufc, int t0) -> bool {
    constexpr int BUF = decltype(bufc)::value;
    const char *Kc = BUF ? Ks1 : Ks0;
    const char *Vc = BUF ? Vs1 : Vs0;
    const bool more = t0 + KB < kend;
    if (more) copy_tile(t0 + KB, BUF ? Ks0 : Ks1, BUF ? Vs0 : Vs1);
    const int nvalid = kend - t0;

    // S^T for two 32-key sub-blocks (rows = keys, columns = this wave's
    // queries), as two interleaved accumulation chains.
    f32x16 s[2];
    s[0] = zero16();
    s[1] = zero16();
#pragma unroll
    for (int c = 0; c < 8; ++c)
#pragma unroll
      for (int sb = 0; sb < 2; ++sb) {
        const bf16x8 a = *(const bf16x8 *)(Kc + sb * 32 * 256 + koff[c]);
        s[sb] = mfma32(a, qop[c], s[sb]);
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
#pragma unroll
    for (int sb = 0; sb < 2; ++sb)
#pragma unroll
      for (int i = 0; i < 16; ++i)
        pb[2 * sb + (i >> 3)][i & 7] = (bf16)exp2_fast(fmaf(s[sb][i], p.scale, -m));
    // Row sums of the rounded probabilities (the values the MFMAs consume).
    float ps[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) ps[kk] = sum_bf16x8(pb[kk], 0.f);
    lsum += (ps[0] + ps[1]) + (ps[2] + ps[3]);

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

    __builtin_amdgcn_s_waitcnt(0);  // this wave's copies of the next tile have landed
    __syncthreads();                // everyone's have, and nobody reads this tile any more
    return more;
  };

  for (int t0 = kbeg;; t0 += 2 * KB) {
    if (!step(std::integral_constant<int, 0>(), t0)) break;
    if (!step(std::integral_constant<int, 1>(), t0 + KB)) break;
  }

  // Partial results: O / l of this key range in bf16, in register order
  // (one 16-byte unit per lane and (bb, r2): elements 4*(2*r2 + e2) + e of
  // o[bb], i.e. d_v = 32bb + 16*r2 + 8*e2 + 4*(l/32) + e), and (m, l) in
  // fp32 per query for the merge.
  const int64_t blk = (((int64_t)b * p.H + h) * p.nqblk + qblk) * p.nsplit + split;
  const float lt = lsum + swap_halves(lsum);
  const float il = 1.f / lt;
  char *wo = p.ws_o + blk * kPartialOBytes + (wave * 8 * 64 + lane) * 16;
#pragma unroll
  for (int bb = 0; bb < 4; ++bb)
#pragma unroll
    for (int r2 = 0; r2 < 2; ++r2) {
      bf16x8 t;
#pragma unroll
      for (int e = 0; e < 8; ++e) t[e] = (bf16)(o[bb][8 * r2 + e] * il);
      *(bf16x8 *)(wo + (2 * bb + r2) * 64 * 16) = t;
    }
  if (hl == 0) {
    float *wml = p.ws_ml + blk * kPartialML + 2 * (wave * 32 + l32);
    wml[0] = m;
    wml[1] = lt;
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
  if (ns > kMaxSplit) ns = kMaxSplit;
  if (ns < 1) ns = 1;
  int64_t kps = (Lk + ns - 1) / ns;
  kps = (kps + kKeyTile - 1) / kKeyTile * kKeyTile;
  pl.kps0 = (int)kps;
  pl.keys_per_split = (int)kps;
  pl.nsplit = (int)((Lk + kps - 1) / kps);
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
  p.kps0 = a.plan.kps0;
  p.kps = a.plan.keys_per_split;
  p.nqblk = a.plan.nqblk;
  p.ws_o = (char *)a.ws_o;
  p.ws_ml = a.ws_ml;
  p.scale = kLog2e / sqrtf((float)D);
  p.nitems = a.B * a.H * a.plan.nsplit * a.plan.nqblk;
  p.per_xcd = (p.nitems + 7) / 8;
  hipLaunchKernelGGL(attn_partial_kernel, dim3((unsigned)(8 * p.per_xcd)), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace arl2
