// The second launch of a pass: the combine (merge of the attention
// partials, the inter-frame read and the output) and, on the clean pass, the
// in-place state update from the chunk contributions that the first launch
// computed (delta_chunk.h). The combine reads only the bf16 copy of the
// pre-update state that the first launch made, so the update of S shares
// the launch.
//
// Method: "Technical Summary: Attend Locally, Remember Linearly (ARL2)",
// section 2.1 (out = O_intra + Q' S_{N-1}; S_N = alpha S_{N-1} +
// K'^T diag(beta)(V' - K' S_{N-1})) and section 2.2 (every token of the frame
// reads the pre-update state; the state is written once per frame, after
// the clean pass). The chunk contributions are summed in a fixed chunk order
// (deterministic, no atomics).
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
  const bf16 *S16;     // bf16 copy of the pre-update state
  int H, L, nqblk, nsplit, nitems;
  bf16 *out;
  const float *o_inter;  // [B][L][H][128] fp32, added when set (and Wq null)
};

// out = (sum_s w_s Ohat_s) / (sum_s w_s) + O_inter with w_s = 2^(m_s - M) l_s,
// Ohat_s = O_s / l_s the normalised partial of key range s and M the largest
// m_s. Lanes own queries and registers own d_v, as in the attention
// kernel's accumulators, so the partials are read in the order they were
// written and O_inter comes out of the MFMAs in the same layout.
// Every load is issued before any arithmetic: bf16(S) and W_q (copied into
// LDS), the queries, the merge weights and the first kPre key ranges'
// partials. The merge runs
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

  // bf16(S)[h] and W_q[h], straight into LDS (swizzled).
  bf16x8 qop[8];
  if (inter) {
    const bf16 *Sh = p.S16 + ((int64_t)b * p.H + h) * D * D;
    const bf16 *W = p.Wq + (int64_t)h * D * D;
    const int r4 = lane >> 4, pos = lane & 15;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int cc = 8 * wave + i, row = 4 * cc + r4;
      const int off = row * D + 8 * (pos ^ tile_swz(row & 15));
      global_to_lds16(Sh + off, St + cc * 1024);
      global_to_lds16(W + off, Wt + cc * 1024);
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
    ss = halves_sum(ss);
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

struct ApplyKParams {
  float *S;
  const float *alpha;
  int arow4;  // 0: one gate per (stream, head); else 4-value groups per d_k row
  const float *ws;
  int nchunk, nitems;
};

// S := gate(S) + sum_c dS_c for 1024 state values of one (stream, head)
// (item = (stream, head, block of 8 rows)), one thread per 4 consecutive
// values; the chunk contributions are summed in chunk order, with up to 16
// loads in flight per thread.
__device__ __forceinline__ void apply_body(const ApplyKParams p, int item) {
  constexpr int dd4 = D * D / 4;
  const int bh = item >> 4;
  const int e = (item & 15) * 256 + threadIdx.x;
  const f32x4 *w = (const f32x4 *)p.ws + (int64_t)bh * p.nchunk * dd4 + e;
  f32x4 *sp = (f32x4 *)p.S + (int64_t)bh * dd4 + e;
  const f32x4 sv = *sp;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int c0 = 0; c0 < p.nchunk; c0 += 16) {
    f32x4 t[16];
#pragma unroll
    for (int u = 0; u < 16; ++u)
      if (c0 + u < p.nchunk) t[u] = w[(int64_t)(c0 + u) * dd4];
#pragma unroll
    for (int u = 0; u < 16; ++u)
      if (c0 + u < p.nchunk) acc += t[u];
  }
  const float a = p.arow4 ? p.alpha[(int64_t)bh * D + e / p.arow4] : p.alpha[bh];
  f32x4 r;
#pragma unroll
  for (int u = 0; u < 4; ++u) r[u] = fmaf(a, sv[u], acc[u]);
  *sp = r;
}

struct TailKParams {
  CombineKParams c;
  ApplyKParams ap;
  int apply_items;  // leading workgroups that apply the state update (0: none)
  int per_xcd_c;
};

// Items of the combine are dealt so that each XCD gets a contiguous run
// (workgroups go to the 8 XCDs round-robin by linear id): the query blocks
// of one head share that XCD's L2 for the head's weights and state. The
// short update items take the first workgroup ids.
__device__ __forceinline__ int xcd_item(int bid, int per_xcd) {
  return (bid & 7) * per_xcd + (bid >> 3);
}

__global__ __launch_bounds__(256, 2) void tail_kernel(TailKParams P) {
  __shared__ __attribute__((aligned(1024))) char lds0[TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char lds1[TILE_BYTES];
  const int bid = blockIdx.x;
  if (bid < P.apply_items) {
    apply_body(P.ap, bid);
  } else {
    const int item = xcd_item(bid - P.apply_items, P.per_xcd_c);
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

hipError_t launch_tail_bf16(const CombineArgs &c, const ApplyArgs *ap, hipStream_t s) {
  TailKParams P;
  P.c.ws_o = (const char *)c.ws_o;
  P.c.ws_ml = c.ws_ml;
  P.c.q = (const bf16 *)c.q;
  P.c.Wq = (const bf16 *)c.Wq;
  P.c.S16 = (const bf16 *)c.S16;
  P.c.H = c.H;
  P.c.L = c.L;
  P.c.nqblk = c.plan.nqblk;
  P.c.nsplit = c.plan.nsplit;
  P.c.nitems = c.B * c.H * c.plan.nqblk;
  P.c.out = (bf16 *)c.out;
  P.c.o_inter = c.Wq ? nullptr : c.o_inter;
  P.per_xcd_c = (P.c.nitems + 7) / 8;
  P.ap = ApplyKParams{};
  P.apply_items = 0;
  if (ap) {
    P.ap.S = ap->S;
    P.ap.alpha = ap->alpha;
    P.ap.arow4 = ap->elementwise ? D / 4 : 0;
    P.ap.ws = ap->ws_dS;
    P.ap.nchunk = ap->nchunk;
    P.ap.nitems = ap->B * ap->H * 16;
    // A multiple of 8, so the combine items keep their XCD runs.
    P.apply_items = (P.ap.nitems + 7) / 8 * 8;
    if (P.apply_items != P.ap.nitems) return hipErrorInvalidValue;
  }
  const unsigned blocks = (unsigned)(P.apply_items + 8 * P.per_xcd_c);
  launch(tail_kernel, dim3(blocks), dim3(256), 0, s, P);
  return hipGetLastError();
}

hipError_t launch_delta_apply(float *S, const float *alpha, bool elementwise, const float *ws_dS,
                              int B, int H, int d, int nchunk, hipStream_t s) {
  const int dd4 = d * d / 4;
  dim3 grid((unsigned)((dd4 + 63) / 64), (unsigned)(B * H));
  launch(delta_apply_kernel, grid, dim3(64), 0, s, S, alpha, elementwise ? d / 4 : 0,
                     ws_dS, dd4, nchunk);
  return hipGetLastError();
}

hipError_t launch_fill_state(float *dst, const float *src, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  dim3 grid((unsigned)((n + 255) / 256));
  launch(fill_state_kernel, grid, dim3(256), 0, s, dst, src, n);
  return hipGetLastError();
}

}  // namespace arl2
