// Internal launch interface between the C ABI (api.hip) and the kernels.
// Not installed; the public interface is include/arl2.h.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace arl2 {

// ---------------------------------------------------------------- launches
// Kernel timing (arl2_profile_enable): while a caller's timing region is
// open on this thread, every launch records the region's `start` event at
// the first kernel's start and its `stop` event at each kernel's end
// (hipExtLaunchKernel events, taken from the kernels' own dispatch), so the
// pair brackets the kernels themselves, with no marker between them.
struct LaunchTiming {
  hipEvent_t start, stop;
  bool started;
};
extern thread_local LaunchTiming *g_launch_timing;

template <class F, class... Args>
inline void launch(F kernel, dim3 grid, dim3 block, uint32_t lds, hipStream_t s, Args... args) {
  if (LaunchTiming *t = g_launch_timing) {
    hipExtLaunchKernelGGL(kernel, grid, block, lds, s, t->started ? nullptr : t->start, t->stop,
                          0, args...);
    t->started = true;
  } else {
    hipLaunchKernelGGL(kernel, grid, block, lds, s, args...);
  }
}

// ---------------------------------------------------------------- plans
// How one attention call is cut into workgroups: query blocks of 128 rows
// (4 wavefronts x 32 queries) and `nsplit` contiguous key ranges: the first
// holds `kps0` keys, the others `keys_per_split` (multiples of the 64-key
// tile). Partial results of the key ranges are merged by the combine kernel.
struct AttnPlan {
  int nqblk = 0;
  int nsplit = 0;
  int kps0 = 0;
  int keys_per_split = 0;
};

constexpr int kQBlock = 128;      // queries per attention workgroup
constexpr int kKeyTile = 64;      // keys per LDS tile
constexpr int kMaxSplit = 8;      // most key ranges one attention call is cut into
constexpr int kGenChunk = 32;     // tokens per delta-update workgroup (generic path)

AttnPlan plan_attention(int64_t B, int64_t H, int64_t Lq, int64_t Lk);

// Partial output per (stream, head, query block, split): O/l for 128
// queries x 128 values in bf16 (in the attention accumulators' register
// order), and (max, sum) per query in fp32.
constexpr int64_t kPartialOBytes = 128 * 128 * 2;
constexpr int64_t kPartialML = 128 * 2;

// ---------------------------------------------------------------- MFMA path
// bf16 io, d = 128.
struct AttnArgs {
  const void *q, *k, *v;  // [B][Lq][H][128], [B][Lk][H][128]
  int B, H, Lq, Lk;
  AttnPlan plan;
  void *ws_o;             // plan blocks x kPartialOBytes
  float *ws_ml;           // plan blocks x kPartialML
};
hipError_t launch_attn_partial_bf16(const AttnArgs &a, hipStream_t s);

// out = merged attention partials + L2norm(q W_q) S (the inter-frame read),
// or the merged partials alone when Wq is null.
struct CombineArgs {
  const void *ws_o;
  const float *ws_ml;
  const void *q;    // [B][L][H][128]
  const void *Wq;   // [H][128][128], or null
  const void *S16;  // [B][H][128][128] bf16 copy of the state (read when Wq is set)
  int B, H, L;
  AttnPlan plan;
  void *out;  // [B][L][H][128] bf16
  const float *o_inter = nullptr;  // [B][L][H][128] fp32, added instead of the read when set
};

// Chunk contributions dS_c of the gated delta update (clean pass).
struct DeltaArgs {
  const void *k, *v;     // [B][L][H][128]
  const void *Wk, *Wv;   // [H][128][128]
  const float *S;        // [B][H][128][128] (pre-update, read only)
  const float *beta;     // [B][L][H]
  int B, H, L;
  int chunk, nchunk;     // tokens per chunk (delta_chunk_tokens), chunks per frame
  float *ws_dS;          // [B][H][nchunk][128][128]
};

// Tokens per delta-update workgroup for a frame of B x H x L: 96 when the
// clean pass's delta chunks and combine items then fit in one round of two
// workgroups per compute unit (shorter items end the launch sooner), else
// 128 (fewer chunk contributions to write and sum).
int delta_chunk_tokens(int64_t B, int64_t H, int64_t L);

// The first launch of a pass: the attention partials, the delta chunks
// when `d` is not null (clean pass), and S16 := bf16(S) for `state_values`
// values (a multiple of 2048) when S is not null. All of them only read S.
hipError_t launch_pass_head_bf16(const AttnArgs &a, const DeltaArgs *d, const float *S, void *S16,
                                 int64_t state_values, hipStream_t s);

// S := gate(S) + sum over chunks c (in order) of ws_dS[b][h][c], as items of
// the second launch of a clean pass (gate as in launch_delta_apply).
struct ApplyArgs {
  float *S;
  const float *alpha;
  bool elementwise;
  const float *ws_dS;
  int B, H, nchunk;
};

// The second launch of a pass: the combine and, when `ap` is not null, the
// state update from the chunk contributions. The combine reads only the
// bf16 copy of the state, so the in-place update can share the launch.
hipError_t launch_tail_bf16(const CombineArgs &c, const ApplyArgs *ap, hipStream_t s);

// ---------------------------------------------------------------- shared
// S[b][h] := gate(S[b][h]) + sum over chunks c (in order) of ws_dS[b][h][c],
// with gate(S) = alpha[b][h] * S (headwise) or row i scaled by
// alpha[b][h][i] (elementwise).
hipError_t launch_delta_apply(float *S, const float *alpha, bool elementwise, const float *ws_dS,
                              int B, int H, int d, int nchunk, hipStream_t s);
// dst[i] := src ? src[i] : 0 for i < n.
hipError_t launch_fill_state(float *dst, const float *src, int64_t n, hipStream_t s);

// ---------------------------------------------------------------- token-level access
constexpr int kTokenChunk = 64;            // tokens per chunk of the recurrence
constexpr int kTokenRecordBytes = 122880;  // MFMA operands of one chunk
struct TokenLevelArgs {
  const void *q, *k, *v;          // [B][L][H][128] bf16
  const void *Wq, *Wk, *Wv;       // [H][128][128] bf16
  const float *alpha, *beta;      // [B][H], [B][L][H]
  float *S;                       // [B][H][128][128], written when update
  int B, H, L, update;
  void *records;                  // [B][H][nchunk] x kTokenRecordBytes
  float *o_inter;                 // [B][L][H][128] fp32
};
// Chunk operands, then the in-order recurrence: O_inter and (update) S.
hipError_t launch_token_level_bf16(const TokenLevelArgs &a, hipStream_t s);
// Any dtype, d in {16, 128}: out = o_intra + O_inter token by token, where
// o_intra is [B][H][L][d] fp32 (the generic attention's layout).
hipError_t launch_token_level_generic(int dtype, int d, const void *q, const void *k,
                                      const void *v, const void *W, const float *o_intra,
                                      float *S, const float *alpha, const float *beta, int B,
                                      int H, int L, int update, void *out, hipStream_t s);

// ---------------------------------------------------------------- gate projections
// Z = x [Wa; Wb]^T on the matrix cores (bf16, D a multiple of 64) or with
// VALU dot products (generic path); beta is written directly, alpha after a
// second launch sums the per-tile alpha logits.
struct GatePlan {
  bool mfma = false;
  int ntt = 0, nnt = 0;  // 16-token tiles, 32-column tiles
  int nta = 0;           // alpha partials per stream (token tiles, or tokens)
  size_t ws_bytes = 0;   // alpha partials [B][nta][H] fp32
};
GatePlan plan_gate(int64_t B, int64_t L, int64_t D, int64_t H, int dtype);

struct GateArgs {
  const void *x;          // [B][L][D]
  const void *Wa, *Wb;    // [H][D]
  int B, L, D, H, dtype;
  GatePlan plan;
  void *ws;               // plan.ws_bytes, 256-byte aligned
  float *alpha, *beta;    // [B][H], [B][L][H]
};
hipError_t launch_gate_projections(const GateArgs &a, hipStream_t s);

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

// Pure bf16 MFMA loop (one 512-thread workgroup per block; `sink` holds
// blocks x 512 floats) and the flops one launch performs.
hipError_t launch_mfma_peak(int blocks, int iters, float *sink, hipStream_t s);
double mfma_peak_flops(int blocks, int iters);

}  // namespace arl2
