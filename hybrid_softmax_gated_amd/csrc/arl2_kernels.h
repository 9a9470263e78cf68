// Internal launch interface between the C ABI (api.hip) and the kernels.
// Not installed; the public interface is include/arl2.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace arl2 {

// ---------------------------------------------------------------- plans
// How one attention call is cut into workgroups: query blocks of 128 rows
// (4 wavefronts x 32 queries) and `nsplit` contiguous key ranges: the first
// holds `kps0` keys, the others `keys_per_split` (multiples of the 64-key
// tile). Partial results of the key ranges are merged by the merge kernel.
struct AttnPlan {
  int nqblk = 0;
  int nsplit = 0;
  int kps0 = 0;
  int keys_per_split = 0;
};

constexpr int kQBlock = 128;      // queries per attention workgroup
constexpr int kKeyTile = 64;      // keys per LDS tile
constexpr int kMaxSplit = 8;      // most key ranges one attention call is cut into
constexpr int kInterKeys = 128;   // keys the first range gives up for the inter-frame read
constexpr int kDeltaChunk = 128;  // tokens per delta-update workgroup (MFMA path)
constexpr int kGenChunk = 32;     // tokens per delta-update workgroup (generic path)

AttnPlan plan_attention(int64_t B, int64_t H, int64_t Lq, int64_t Lk, bool inter);

// Elements of partial output per (stream, head, query block, split):
// O/l[128][128] (bf16, in a slot sized for fp32) and (max, sum)[128] (fp32).
constexpr int64_t kPartialO = 128 * 128;
constexpr int64_t kPartialML = 128 * 2;

// ---------------------------------------------------------------- MFMA path
// bf16 io, d = 128.
struct AttnArgs {
  const void *q, *k, *v;  // [B][Lq][H][128], [B][Lk][H][128]
  const void *Wq;         // [H][128][128] (read when ws_inter is set)
  const float *S;         // [B][H][128][128] (read when ws_inter is set)
  int B, H, Lq, Lk;
  AttnPlan plan;
  float *ws_o, *ws_ml;
  float *ws_inter;        // [B][H][nqblk*128][128] O_inter, or null for plain attention
};
hipError_t launch_attn_partial_bf16(const AttnArgs &a, hipStream_t s);

struct MergeArgs {
  const float *ws_o, *ws_ml, *ws_inter;  // ws_inter may be null
  int B, H, L;
  AttnPlan plan;
  void *out;  // [B][L][H][128] bf16
};
hipError_t launch_merge_bf16(const MergeArgs &a, hipStream_t s);

struct DeltaArgs {
  const void *k, *v;     // [B][L][H][128]
  const void *Wk, *Wv;   // [H][128][128]
  const float *S;        // [B][H][128][128] (pre-update, read only)
  const float *beta;     // [B][L][H]
  int B, H, L, nchunk;
  float *ws_dS;          // [B][H][nchunk][128][128]
};
hipError_t launch_delta_partial_bf16(const DeltaArgs &a, hipStream_t s);

// ---------------------------------------------------------------- shared
// S[b][h] := alpha[b][h] * S[b][h] + sum over chunks c (in order) of
// ws_dS[b][h][c], elementwise.
hipError_t launch_delta_apply(float *S, const float *alpha, const float *ws_dS, int B, int H,
                              int d, int nchunk, hipStream_t s);
// dst[i] := src ? src[i] : 0 for i < n.
hipError_t launch_fill_state(float *dst, const float *src, int64_t n, hipStream_t s);

// ---------------------------------------------------------------- generic path
// Any dtype, d in {16, 128}: plain VALU kernels for the small fp32 workloads.
// dtype: 0 = bf16, 1 = f32 (arl2_dtype).
hipError_t launch_generic_attention(int dtype, int d, const void *q, const void *k, const void *v,
                                    int B, int H, int Lq, int Lk, float *o_intra, hipStream_t s);
hipError_t launch_generic_inter_combine(int dtype, int d, const void *q, const void *Wq,
                                        const float *S, const float *o_intra, int B, int H, int L,
                                        void *out, bool with_inter, hipStream_t s);
hipError_t launch_generic_delta_partial(int dtype, int d, const void *k, const void *v,
                                        const void *Wk, const void *Wv, const float *S,
                                        const float *beta, int B, int H, int L, float *ws_dS,
                                        hipStream_t s);

}  // namespace arl2
