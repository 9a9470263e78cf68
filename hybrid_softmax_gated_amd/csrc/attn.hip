// The first launch of a pass (bf16 io, d = 128): intra-frame softmax
// attention on the gfx950 matrix cores, written as partial results per key
// range; on a clean pass also the chunk contributions of the gated delta
// state update (delta_chunk.h); and a bf16 copy of the state for the
// inter-frame read of the second launch.
//
// Method: "Technical Summary: Attend Locally, Remember Linearly (ARL2)",
// section 2.1 — the intra-frame branch keeps full bidirectional softmax
// attention inside the frame; the inter-frame branch reads the fixed-size
// state with feature-mapped, L2-normalised queries; section 2.2 — every token
// of the frame reads the same pre-update state, and only the clean pass
// writes it.
//
// Data layout in HBM: q, k, v, out are token-major [B][L][H][128] bf16, so a
// head's row of 128 values is 256 contiguous bytes and consecutive tokens of
// one head are H*256 bytes apart.
//
// Attention items (one contiguous key range of one head; in the launch of
// a clean pass 4 wavefronts = one block of 128 queries per workgroup, two
// workgroups per compute unit, beside the update chunks; in every other
// launch 8 wavefronts = two blocks of 128 queries sharing each K/V tile,
// one workgroup per compute unit):
//  * each wavefront keeps its 32 queries in registers as MFMA B operands and
//    computes the transposed score tile S^T = K Q^T (keys on rows), so every
//    lane owns one query: the row max and row sum of the online softmax are
//    in-register reductions plus one VALU lane swap between the wave halves;
//  * K and V tiles of 64 keys are staged in LDS row-major with a 16-byte
//    XOR swizzle (no bank conflicts for either read pattern); V is read as
//    the A operand of O^T = V^T P^T with the LDS transpose read, in the key
//    order that lets the softmax probabilities leave the score accumulators
//    and enter the next MFMA as its B operand with no data movement;
//  * double-buffered tiles: the next tile's buffer->LDS copies are issued
//    before the current tile's MFMAs and waited for at the tile's end (one
//    barrier per tile); the first tile waits only for its K copies before
//    its scores and for its V copies before P.V; the loop is unrolled by two
//    so every LDS address is a constant offset from a per-lane register;
//  * per key range it writes O/l in bf16, in the accumulators' register
//    order (16-byte coalesced stores), and the row max (log2 domain) and row
//    sum in fp32.
// Update chunks and state-copy items take the workgroup ids after the
// attention items; all three only read the state, so they share the launch.
#include "arl2_device.h"
#include "arl2_kernels.h"
#include "delta_chunk.h"

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

// One attention item of a workgroup of NW wavefronts. NW = 4: one block of
// 128 queries (item = stream, head, key range, query block). NW = 8: two
// consecutive blocks over the same key range (item = stream, head, key
// range, pair of blocks); wavefronts 4-7 take the second block, and all
// eight share every K/V tile, which halves the tile copies per query.
// Ks0/Ks1/Vs0/Vs1: double-buffered K and V tiles, each its own LDS array so
// that the compiler sees the copies into one buffer and the reads of the
// other as disjoint.
template <int NW>
__device__ __forceinline__ void attn_body(const AttnKParams &p, int item, char *Ks0, char *Ks1,
                                          char *Vs0, char *Vs1) {
  static_assert(NW == 4 || NW == 8, "wavefronts per workgroup");
  const int nunit = NW == 4 ? p.nqblk : (p.nqblk + 1) / 2;
  const int unit = item % nunit;
  int rest = item / nunit;
  const int split = rest % p.nsplit;
  rest /= p.nsplit;
  const int h = rest % p.H, b = rest / p.H;

  const int tid = threadIdx.x;
  const int waveN = tid >> 6, lane = tid & 63, hl = lane >> 5, l32 = lane & 31;
  const int wave = NW == 4 ? waveN : waveN & 3;  // wavefront within its query block
  const int qblk = NW == 4 ? unit : 2 * unit + (waveN >> 2);
  // The second block of the last pair may lie past the frame: its
  // wavefronts still copy tiles and meet every barrier, on zero queries.
  const bool active = NW == 4 || qblk < p.nqblk;
  const int64_t tok = (int64_t)p.H * D;     // elements between tokens
  const int64_t tokB = tok * 2;             // bytes between tokens
  const bf16 *qbase = p.q + ((int64_t)b * p.Lq * p.H + h) * D;
  const char *kbase = (const char *)(p.k + ((int64_t)b * p.Lk * p.H + h) * D);
  const char *vbase = (const char *)(p.v + ((int64_t)b * p.Lk * p.H + h) * D);
  const int kbeg = split == 0 ? 0 : p.kps0 + (split - 1) * p.kps;
  const int kend = min(p.Lk, split == 0 ? p.kps0 : kbeg + p.kps);

  // Tile copies: the 16 chunks of 4 rows (1 KB) of a tile are shared out,
  // CPW = 16 / NW per wavefront (chunks CPW*w .. CPW*w + CPW-1); lane
  // (r4 = l/16, pos = l%16) of chunk cc fetches row 4cc + r4, 16-byte unit
  // pos ^ swizzle, so the bytes land in the swizzled layout.
  constexpr int CPW = 16 / NW;
  int doff[CPW];
#pragma unroll
  for (int i = 0; i < CPW; ++i) {
    const int row = 4 * (CPW * waveN + i) + (lane >> 4);
    doff[i] = (int)(row * tokB) + 16 * ((lane & 15) ^ tile_swz(row & 15));
  }
  // Copy the K (or V) rows of the tile starting at key t0 into kt (vt):
  // CPW loads per wavefront; rows at or past kend read as zeros.
  // Bytes of K (or V) rows from key t0 to kend: 0 when t0 >= kend, so that
  // a copy past the range issues its loads but reads nothing.
  auto tile_bytes = [&](int t0) {
    const int64_t span = (int64_t)(kend - t0) * tokB;
    return (uint32_t)(span <= 0 ? (int64_t)0 : span < (int64_t)0x7fffffff ? span : (int64_t)0x7fffffff);
  };
  auto copy_rows = [&](const char *base, int t0, char *dst) {
    const __amdgpu_buffer_rsrc_t r = make_rsrc(base + t0 * tokB, tile_bytes(t0));
#pragma unroll
    for (int i = 0; i < CPW; ++i) buffer_to_lds16(r, dst + (CPW * waveN + i) * 1024, doff[i]);
  };
  auto copy_tile = [&](int t0, char *kt, char *vt) {
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(kbase + t0 * tokB, tile_bytes(t0));
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(vbase + t0 * tokB, tile_bytes(t0));
#pragma unroll
    for (int i = 0; i < CPW; ++i) {
      buffer_to_lds16(rk, kt + (CPW * waveN + i) * 1024, doff[i]);
      buffer_to_lds16(rv, vt + (CPW * waveN + i) * 1024, doff[i]);
    }
  };

  // Loads of the first tile, in the order they are waited for: K (CPW
  // copies), the wavefront's 32 queries (8 loads), V (CPW copies). Every
  // wavefront issues all of them, so the in-order load counter tells
  // when each group has landed. The queries become B operands: lane l
  // holds query l%32, head-dim elements 16c + 8*(l/32) .. +7 (zeros past
  // the frame).
  copy_rows(kbase, kbeg, Ks0);
  __builtin_amdgcn_sched_barrier(0);  // keep the three groups in this order
  const int qrow0 = qblk * kQBlock + wave * 32;
  const int qrows = max(0, min(32, p.Lq - qrow0));
  const __amdgpu_buffer_rsrc_t rq =
      make_rsrc(qbase + (int64_t)qrow0 * tok, (uint32_t)qrows * (uint32_t)tokB);
  bf16x8 qop[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) qop[c] = buffer_load16(rq, l32 * (int)tokB + 32 * c + 16 * hl);
  __builtin_amdgcn_sched_barrier(0);
  copy_rows(vbase, kbeg, Vs0);

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

  // Every wavefront's K copies of the first tile have landed; its queries
  // and V copies may still be in flight.
  vm_barrier<8 + CPW>();

  // One 64-key tile from buffer BUF; the next tile is copied into the other
  // buffer meanwhile. Returns false after the last tile.
  auto step = [&](auto bufc, auto firstc, int t0) -> bool {
    constexpr int BUF = decltype(bufc)::value;
    constexpr bool FIRST = decltype(firstc)::value;
    const char *Kc = BUF ? Ks1 : Ks0;
    const char *Vc = BUF ? Vs1 : Vs0;
    const bool more = t0 + KB < kend;
    // The first tile always issues the next copy (of zero rows if there is
    // no next tile), so the number of loads in flight behind its own V
    // copies does not depend on the range.
    if (FIRST || more) copy_tile(t0 + KB, BUF ? Ks0 : Ks1, BUF ? Vs0 : Vs1);
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
    mx = halves_max(mx) * p.scale;
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

    // Probabilities, rounded to bf16 for the MFMAs; the row sums add the
    // fp32 values with plain VALU adds. (The bf16 dot-product instruction
    // would sum the rounded values in half the instructions, but on gfx950
    // it waits for the SIMD's matrix core, which the other wavefront keeps
    // busy.) The two sums differ by at most 2^-9 relative, the bf16
    // rounding step of the output itself, and by much less when many keys
    // contribute (round-to-nearest-even errors have no bias).
    bf16x8 pb[4];
    float ps[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int sb = 0; sb < 2; ++sb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float e = exp2_fast(fmaf(s[sb][i], p.scale, -m));
        pb[2 * sb + (i >> 3)][i & 7] = (bf16)e;
        ps[2 * sb + (i >> 3)] += e;
      }
    lsum += (ps[0] + ps[1]) + (ps[2] + ps[3]);

    // The first tile's V copies of every wavefront have landed (the next
    // tile's 2*CPW copies may not).
    if constexpr (FIRST) vm_barrier<2 * CPW>();

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

  // The first tile has its own copy of the loop body, so that only its
  // code waits for the queries and V copies one by one; the loop proper
  // starts with everything landed.
  using B0 = std::integral_constant<int, 0>;
  using B1 = std::integral_constant<int, 1>;
  using First = std::true_type;
  using Later = std::false_type;
  if (step(B0(), First(), kbeg)) {
    for (int t0 = kbeg + KB;; t0 += 2 * KB) {
      if (!step(B1(), Later(), t0)) break;
      if (!step(B0(), Later(), t0 + KB)) break;
    }
  }

  if (!active) return;
  // Partial results: O / l of this key range in bf16, in register order
  // (one 16-byte unit per lane and (bb, r2): elements 4*(2*r2 + e2) + e of
  // o[bb], i.e. d_v = 32bb + 16*r2 + 8*e2 + 4*(l/32) + e), and (m, l) in
  // fp32 per query for the merge.
  const int64_t blk = (((int64_t)b * p.H + h) * p.nqblk + qblk) * p.nsplit + split;
  const float lt = halves_sum(lsum);
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

// S16 := bf16(S) (round to nearest even) for 8 * NT state values per item
// (NT threads per workgroup).
template <int NT>
__device__ __forceinline__ void state_copy_body(const float *S, bf16 *S16, int item) {
  const int64_t i0 = ((int64_t)item * NT + threadIdx.x) * 8;
  const f32x4 a = *(const f32x4 *)(S + i0);
  const f32x4 c = *(const f32x4 *)(S + i0 + 4);
  bf16x8 t;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    t[e] = (bf16)a[e];
    t[4 + e] = (bf16)c[e];
  }
  *(bf16x8 *)(S16 + i0) = t;
}

struct PassKParams {
  AttnKParams a;
  DeltaKParams d;
  const float *S;   // state to copy (null: no copy items)
  bf16 *S16;
  int attn_blocks;  // workgroups of attention items (8 * per_xcd)
  int delta_blocks; // workgroups of update chunks (8 * per_xcd_d)
  int per_xcd_d;
  int copy_items;
};

// Workgroups [0, attn_blocks): attention; then the update chunks (dealt to
// XCDs in contiguous runs, so one head's chunks share an L2 for its weights
// and state); then the state copy.
template <int NT>
__global__ __launch_bounds__(256, 2) void pass_head_kernel(PassKParams P) {
  __shared__ __attribute__((aligned(1024))) char Ks0[TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char Ks1[TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char Vs0[TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char Vs1[TILE_BYTES];
  __shared__ float betas[32 * 4];
  int bid = blockIdx.x;
  if (bid < P.attn_blocks) {
    const int item = item_of(bid, P.a.per_xcd);
    if (item < P.a.nitems) attn_body<4>(P.a, item, Ks0, Ks1, Vs0, Vs1);
    return;
  }
  bid -= P.attn_blocks;
  if (bid < P.delta_blocks) {
    const int item = item_of(bid, P.per_xcd_d);
    if (item < P.d.nitems)
      delta_body<NT>(P.d, item, SplitTile{Ks0, Ks1}, SplitTile{Vs0, Vs1}, betas);
    return;
  }
  bid -= P.delta_blocks;
  if (bid < P.copy_items) state_copy_body<256>(P.S, P.S16, bid);
}

// A launch with no update chunks (query-only passes, attention over a key
// cache): eight wavefronts per workgroup, two query blocks per attention
// item, one workgroup per compute unit; then the state copy, 4096 values
// per workgroup.
__global__ __launch_bounds__(512, 1) void attn8_kernel(PassKParams P) {
  __shared__ __attribute__((aligned(1024))) char Ks0[TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char Ks1[TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char Vs0[TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char Vs1[TILE_BYTES];
  int bid = blockIdx.x;
  if (bid < P.attn_blocks) {
    const int item = item_of(bid, P.a.per_xcd);
    if (item < P.a.nitems) attn_body<8>(P.a, item, Ks0, Ks1, Vs0, Vs1);
    return;
  }
  bid -= P.attn_blocks;
  if (bid < P.copy_items) state_copy_body<512>(P.S, P.S16, bid);
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

// Kernel parameters of the attention items, for workgroups of NW wavefronts.
static AttnKParams attn_params(const AttnArgs &a, int nw) {
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
  const int units = nw == 4 ? a.plan.nqblk : (a.plan.nqblk + 1) / 2;
  p.nitems = a.B * a.H * a.plan.nsplit * units;
  p.per_xcd = (p.nitems + 7) / 8;
  return p;
}

hipError_t launch_pass_head_bf16(const AttnArgs &a, const DeltaArgs *d, const float *S, void *S16,
                                 int64_t state_values, hipStream_t s) {
  if (d && d->chunk != 96 && d->chunk != 128) return hipErrorInvalidValue;
  PassKParams P;
  if (!d) {
    // No update chunks: the eight-wavefront kernel.
    if (S && state_values % 4096 != 0) return hipErrorInvalidValue;
    P.a = attn_params(a, 8);
    P.attn_blocks = 8 * P.a.per_xcd;
    P.d = DeltaKParams{};
    P.delta_blocks = 0;
    P.per_xcd_d = 0;
    P.S = S;
    P.S16 = (bf16 *)S16;
    P.copy_items = S ? (int)(state_values / 4096) : 0;
    launch(attn8_kernel, dim3((unsigned)(P.attn_blocks + P.copy_items)), dim3(512), 0, s, P);
    return hipGetLastError();
  }
  if (S && state_values % 2048 != 0) return hipErrorInvalidValue;
  // With update chunks: four-wavefront workgroups, two per compute unit.
  P.a = attn_params(a, 4);
  P.attn_blocks = 8 * P.a.per_xcd;
  P.d = DeltaKParams{};
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
  P.S = S;
  P.S16 = (bf16 *)S16;
  P.copy_items = S ? (int)(state_values / 2048) : 0;
  const unsigned blocks = (unsigned)(P.attn_blocks + P.delta_blocks + P.copy_items);
  if (d->chunk == 96)
    launch(pass_head_kernel<3>, dim3(blocks), dim3(256), 0, s, P);
  else
    launch(pass_head_kernel<4>, dim3(blocks), dim3(256), 0, s, P);
  return hipGetLastError();
}

hipError_t launch_attn_partial_bf16(const AttnArgs &a, hipStream_t s) {
  return launch_pass_head_bf16(a, nullptr, nullptr, nullptr, 0, s);
}

}  // namespace arl2
