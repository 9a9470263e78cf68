/*
 * libarl2 — one ARL2 ("Attend Locally, Remember Linearly") hybrid attention
 * layer on AMD Instinct MI355X (gfx950).
 *
 * The method (see "Technical Summary: Attend Locally, Remember Linearly
 * (ARL2)", gist.science, section 2.1 "Hybrid Attention Decomposition" and
 * section 2.2 "Memory State Management") splits a video DiT's self-attention
 * into two branches per head:
 *
 *   intra-frame: softmax attention among the L tokens of the current frame,
 *                bidirectional (no mask), scale 1/sqrt(d);
 *   inter-frame: a fixed-size state S (d_k x d_v, fp32, per stream and head)
 *                read through feature-mapped queries, O_inter = Q' S_{N-1},
 *                and written once per frame by the gated delta rule
 *                S_N = alpha S_{N-1} + K'^T diag(beta) (V' - K' S_{N-1}).
 *
 * Q' = L2norm(q W_q), K' = L2norm(k W_k), V' = v W_v (per-head d x d maps,
 * row-vector convention x' = x W, no bias; the L2 normalisation, with a
 * 1e-6 floor on the norm, is this library's choice — the pages do not state
 * one). The layer output is the plain sum out = O_intra + O_inter.
 * Every token of a frame reads the same pre-update state (frame-level
 * access); noisy denoising passes only read S, and only the final clean pass
 * of a frame updates it (clean-pass updates).
 *
 * Conventions for every entry point:
 *  - All tensor pointers are DEVICE pointers owned by the caller. The
 *    layer's entry points never allocate device memory (only the measurement
 *    call arl2_profile_mfma_peak takes and frees a small buffer of its own);
 *    the library never frees caller memory and keeps no pointer beyond the
 *    arl2_state descriptor the caller owns.
 *  - Activations use token-major layout [B][L][H][d], contiguous.
 *  - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *    Work is enqueued asynchronously; kernel faults surface at the caller's
 *    next synchronisation of that stream.
 *  - Every argument is validated before anything is enqueued. On any error
 *    nothing is written and nothing is launched.
 *  - Calls on different states may run concurrently on different streams.
 *    Two calls that share one state (its S or its workspace) must be
 *    ordered by the caller (same stream, or events).
 *  - Results are bitwise reproducible run to run: no floating-point atomics.
 *  - The compute entry points only launch kernels on `stream` (no memsets,
 *    no host synchronisation, no allocation), so a caller may capture them
 *    into a HIP graph and replay it; a replay gives the bytes the same calls
 *    give eagerly. Kernel timing (arl2_profile_enable) is the exception.
 */
#ifndef ARL2_H
#define ARL2_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#if defined(__GNUC__)
#define ARL2_API __attribute__((visibility("default")))
#else
#define ARL2_API
#endif

#define ARL2_VERSION 1

typedef enum {
  ARL2_OK = 0,
  ARL2_ERR_INVALID_ARG = 1, /* NULL/misaligned pointer, bad size or flag     */
  ARL2_ERR_UNSUPPORTED = 2, /* a valid request the library does not handle   */
  ARL2_ERR_HIP = 3          /* the HIP runtime refused a launch or a copy    */
} arl2_status;

typedef enum {
  ARL2_BF16 = 0, /* q, k, v, W_phi, out stored as bfloat16 */
  ARL2_F32 = 1   /* q, k, v, W_phi, out stored as float32  */
} arl2_dtype;

/* Head dimensions the library supports (d_k = d_v = d). */
#define ARL2_D_SMALL 16
#define ARL2_D_LARGE 128

/* Largest tokens-per-frame value accepted (keeps every index in int32). */
#define ARL2_MAX_L (1 << 20)

/*
 * Per-layer state descriptor. Plain data; the caller owns it and the buffers
 * it points to. Filled by arl2_state_init; do not modify its fields after.
 */
typedef struct {
  int32_t B;        /* independent streams (batch)                          */
  int32_t H;        /* heads                                                 */
  int32_t d;        /* head dimension: 16 or 128                             */
  int32_t L;        /* tokens per frame (fixed for the life of the state)    */
  int32_t dtype;    /* arl2_dtype of the io tensors                          */
  int32_t magic;    /* set by arl2_state_init; marks the descriptor as bound */
  float *S;         /* device, [B][H][d][d] fp32, row = d_k, column = d_v    */
  void *ws;         /* device workspace of ws_bytes bytes                    */
  size_t ws_bytes;
} arl2_state;

/*
 * Bytes of device workspace arl2_frame_forward needs for this shape.
 * Returns 0 for an invalid shape. The workspace holds partial results of the
 * split attention and of the split state update between kernels; its size
 * does not depend on the number of frames.
 */
ARL2_API size_t arl2_workspace_bytes(int32_t B, int32_t H, int32_t d, int32_t L, int32_t dtype);

/*
 * Bind a state to caller-owned device memory and set S := 0.
 * The state is the fixed-size d_k x d_v matrix per stream and head that the
 * inter-frame branch carries from frame to frame ("Technical Summary ...",
 * section 2.2 "Memory State Management": its size does not grow with the
 * number of frames, which is where the constant memory of section 4 comes
 * from); a new stream starts from the empty memory S = 0.
 *   S_dev   device [B][H][d][d] float32, 16-byte aligned.
 *   ws_dev  device workspace of at least arl2_workspace_bytes(...) bytes,
 *           256-byte aligned; or NULL with ws_bytes == 0 for a state whose
 *           passes all go through arl2_frame_forward_noalloc (the other
 *           pass entry points then return INVALID_ARG for it).
 * The zero fill is enqueued on `stream`.
 * Errors: INVALID_ARG for NULL st/S_dev, a bad shape, a too-small or
 * misaligned workspace; UNSUPPORTED for d not in {16, 128}.
 */
ARL2_API arl2_status arl2_state_init(arl2_state *st, int32_t B, int32_t H, int32_t d, int32_t L,
                            int32_t dtype, float *S_dev, void *ws_dev, size_t ws_bytes,
                            void *stream);

/*
 * Start a new video stream on an initialised state: S := S0 (device,
 * [B][H][d][d] float32, may not alias S), or S := 0 when S0_dev is NULL.
 * Restoring a saved S this way resumes a stream exactly where it was: the
 * state is all the inter-frame branch remembers of earlier frames
 * ("Technical Summary ...", section 2.2), so S plus the next frame's
 * inputs determine everything that follows.
 * Errors: INVALID_ARG for a state not set up by arl2_state_init, or an S0
 * that is misaligned (4 bytes) or overlaps S; ARL2_ERR_HIP if the copy
 * kernel cannot be launched.
 */
ARL2_API arl2_status arl2_state_reset(arl2_state *st, const float *S0_dev, void *stream);

/*
 * One pass of one frame through the layer ("Technical Summary ...", section
 * 2.1 "Hybrid Attention Decomposition": out = softmax attention inside the
 * frame + Q' S_{N-1}; section 2.2 "Memory State Management": every token of
 * the frame reads the same pre-update state, and only the final clean pass
 * of a frame writes S_N = alpha S_{N-1} + K'^T diag(beta) (V' - K' S_{N-1}),
 * so the denoising passes in between leave S untouched).
 *   q, k, v  device [B][L][H][d], io dtype, 16-byte aligned, not aliasing out.
 *   Wphi     device [3][H][d][d], io dtype: the maps for q, k, v; map[m][h]
 *            is stored [d_in][d_out] and applied as x' = x W.
 *   st       state from arl2_state_init (shape taken from it).
 *   alpha    device [B][H] float32: this frame's forget gate, one scalar per
 *            stream and head. Read only when update_flag == 1 (may be NULL
 *            when update_flag == 0).
 *   beta     device [B][L][H] float32: this frame's per-token learning rate.
 *            Same NULL rule as alpha.
 *   out      device [B][L][H][d], io dtype: O_intra + O_inter, rounded to the
 *            io dtype (round to nearest even).
 *   update_flag 0 = noisy (query-only) pass: S is not touched.
 *               1 = clean pass: out is computed from the pre-update S, then
 *                   S is updated in place, in stream order.
 * Errors: INVALID_ARG for NULL/misaligned pointers, aliasing of out with an
 * input, the state or its workspace (and, when update_flag == 1, with alpha
 * or beta), inputs overlapping the state or its workspace, update_flag not
 * in {0, 1}, NULL alpha/beta with update_flag == 1, or an uninitialised
 * state; ARL2_ERR_HIP if a launch fails.
 */
ARL2_API arl2_status arl2_frame_forward(const void *q, const void *k, const void *v, const void *Wphi,
                               arl2_state *st, const float *alpha, const float *beta,
                               void *out, int32_t update_flag, void *stream);

/*
 * arl2_frame_forward without a caller workspace, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation). The pass's partial results live
 * in a scratch array of ARL2_NOALLOC_SCRATCH_BYTES that the library holds
 * on each device it runs on until the process ends; the call allocates
 * nothing and frees nothing. The state may have been bound with or without
 * a workspace (arl2_state_init); its own workspace is not used.
 *   Arguments, layout, ownership and results are those of
 *   arl2_frame_forward (headwise gate).
 * Every call on one device shares that device's scratch: calls that may
 * overlap in time on one device (different streams, or different host
 * threads without ordering) race on it and must be ordered by the caller.
 * The scratch keeps the last call's contents; nothing in it needs to start
 * at zero.
 * Errors: those of arl2_frame_forward; INVALID_ARG also when the state's
 * shape needs more than ARL2_NOALLOC_SCRATCH_BYTES of scratch
 * (arl2_workspace_bytes tells how much it needs); ARL2_ERR_HIP if the
 * scratch's device address cannot be found.
 */
#define ARL2_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
ARL2_API arl2_status arl2_frame_forward_noalloc(const void *q, const void *k, const void *v,
                                                const void *Wphi, arl2_state *st,
                                                const float *alpha, const float *beta, void *out,
                                                int32_t update_flag, void *stream);

/* Forget-gate kinds of arl2_frame_forward_gated. */
typedef enum {
  ARL2_GATE_HEADWISE = 0,   /* alpha [B][H]: one scalar per stream, head and frame       */
  ARL2_GATE_ELEMENTWISE = 1 /* alpha [B][H][d]: one value per d_k row of the state      */
} arl2_gate;

/*
 * arl2_frame_forward with a choice of forget gate. The pages' ablation
 * ("Technical Summary ...", section 4 "Experimental Results", Ablations;
 * atlas.scime.ai summary, "Surprising findings") compares the method's
 * headwise gate with elementwise gating and prints no formula for the
 * latter; this library reads it as one gate per key channel:
 *   S_N = diag(alpha) S_{N-1} + K'^T diag(beta) (V' - K' S_{N-1}),
 * i.e. row i (d_k index) of the carried state is scaled by alpha[b][h][i];
 * the residual reads the ungated S_{N-1}.
 *   gate   ARL2_GATE_HEADWISE: alpha is device [B][H] float32 and the call is
 *          exactly arl2_frame_forward. ARL2_GATE_ELEMENTWISE: alpha is device
 *          [B][H][d] float32.
 * Every other argument, the layout, ownership and the errors are those of
 * arl2_frame_forward; a gate outside arl2_gate is INVALID_ARG.
 */
ARL2_API arl2_status arl2_frame_forward_gated(const void *q, const void *k, const void *v,
                                     const void *Wphi, arl2_state *st, const float *alpha,
                                     int32_t gate, const float *beta, void *out,
                                     int32_t update_flag, void *stream);

/*
 * One pass with token-level state access: the ablation that frame-level
 * access is compared with ("Technical Summary ...", section 4; frame-level
 * access is section 2.2). The pages only name it; the reading here: inside
 * the frame the tokens write the state one after another and each token's
 * query reads it right after its own write,
 *   S_1 = alpha S_0 + beta_1 k'_1 (v'_1 - k'_1^T S_0),
 *   S_i = S_{i-1} + beta_i k'_i (v'_i - k'_i^T S_{i-1})  (i > 1),
 *   out[i] = O_intra[i] + q'_i S_i,
 * with the forget gate applied once per frame, with the first token (a
 * one-token frame is the frame-level update). Clean-pass updates still hold:
 * update_flag = 0 forms the within-frame states for the reads only and
 * leaves S bitwise unchanged; update_flag = 1 stores S_L.
 * Arguments as for arl2_frame_forward (headwise alpha [B][H]), except:
 *   alpha, beta  required on every pass;
 *   tl_ws        device workspace of arl2_token_level_workspace_bytes(...)
 *                bytes, 256-byte aligned, contents need not be initialised
 *                (the size is 0, and tl_ws may be NULL, for shapes other than
 *                bf16 with d = 128, which run token by token).
 * Errors: as arl2_frame_forward, plus INVALID_ARG for NULL alpha/beta, a
 * short or misaligned tl_ws, or tl_ws overlapping any other buffer.
 */
ARL2_API size_t arl2_token_level_workspace_bytes(int32_t B, int32_t H, int32_t d, int32_t L,
                                                 int32_t dtype);
ARL2_API arl2_status arl2_frame_forward_token_level(const void *q, const void *k, const void *v,
                                                    const void *Wphi, arl2_state *st,
                                                    const float *alpha, const float *beta,
                                                    void *out, int32_t update_flag, void *tl_ws,
                                                    size_t tl_ws_bytes, void *stream);

/*
 * Full-softmax attention of Lq queries over Lk cached keys/values per stream
 * and head, with scale 1/sqrt(d) and no mask: the growing key/value-cache
 * attention that the method replaces ("Technical Summary ...", section 1,
 * KV cache growth). Same kernels as the intra-frame branch.
 *   q   device [B][Lq][H][d];  kc, vc device [B][Lk][H][d];  out [B][Lq][H][d]
 *   ws  device workspace of arl2_softmax_attention_workspace_bytes(...) bytes.
 */
ARL2_API size_t arl2_softmax_attention_workspace_bytes(int32_t B, int32_t H, int32_t d, int32_t Lq,
                                              int32_t Lk, int32_t dtype);
ARL2_API arl2_status arl2_softmax_attention(const void *q, const void *kc, const void *vc, int32_t B,
                                   int32_t H, int32_t d, int32_t Lq, int32_t Lk, int32_t dtype,
                                   void *out, void *ws, size_t ws_bytes, void *stream);

/*
 * Gate projections: the delta rule's gates computed from the tokens that
 * enter the layer ("Technical Summary ...", section 2.1: alpha and beta are
 * learned per-token projections; section 4, ablations: the forget gate is
 * headwise). With z_a = x . Wa[h] and z_b = x . Wb[h] per token:
 *   beta[b][t][h] = sigmoid(x[b][t] . Wb[h])          one per token and head
 *   alpha[b][h]   = sigmoid(mean_t x[b][t] . Wa[h])   one per stream, head, frame
 * The pages do not state how per-token forget gates become the one headwise
 * gate a frame-level update applies; this library pools the logits by their
 * mean over the frame's L tokens. No bias. The outputs are laid out as the
 * alpha and beta arguments of arl2_frame_forward take them.
 *   x      device [B][L][D] in `dtype`: the frame's tokens entering the layer
 *   Wa, Wb device [H][D] in `dtype`: one row of D weights per head (the
 *          weight layout of a linear map from D to H features)
 *   alpha  device [B][H] float32 (written)
 *   beta   device [B][L][H] float32 (written)
 *   ws     device workspace of arl2_gate_projections_workspace_bytes(...)
 *          bytes, 256-byte aligned; contents need not be initialised.
 * Sums are in fp32; bf16 inputs with D a multiple of 64 use the matrix cores.
 * Errors: INVALID_ARG for a bad dtype or shape (B, L, H >= 1, 1 <= D <=
 * ARL2_MAX_GATE_D), NULL or misaligned pointers (x, Wa, Wb 16 bytes; alpha,
 * beta 4 bytes), a short workspace, or outputs that overlap the inputs or
 * each other. The workspace-size query returns 0 for a bad shape.
 */
#define ARL2_MAX_GATE_D (1 << 16)
ARL2_API size_t arl2_gate_projections_workspace_bytes(int32_t B, int32_t L, int32_t D, int32_t H,
                                                      int32_t dtype);
ARL2_API arl2_status arl2_gate_projections(const void *x, const void *Wa, const void *Wb,
                                           int32_t B, int32_t L, int32_t D, int32_t H,
                                           int32_t dtype, float *alpha, float *beta, void *ws,
                                           size_t ws_bytes, void *stream);

/*
 * Kernel timing (diagnostics). While enabled, every launch (or pair of
 * launches that one call makes for one step) is timed with a pair of
 * hipEvents. With repeat = 1 the events are taken from the kernels' own
 * start and end (hipExtLaunchKernel), so a time is that of the launch in its
 * place in the call sequence, with no marker in between. With repeat > 1 a
 * launch that only reads its inputs and overwrites its outputs (all but the
 * in-place state update) is issued `repeat` times back to back between two
 * event markers, which spreads the markers' own overhead over the repeats;
 * the results are those of a single launch. arl2_profile_report waits for
 * the recorded events and writes one line per launch kind,
 * "<name> <launches> <total_ms>\n", into buf (NUL-terminated, truncated to
 * len). Disabled by default. Not for use under graph capture.
 * Errors: INVALID_ARG for repeat outside [1, 1000], a NULL buf or len 0;
 * ARL2_ERR_HIP if an event cannot be created or queried.
 */
ARL2_API arl2_status arl2_profile_enable(int32_t on, int32_t repeat);
ARL2_API arl2_status arl2_profile_report(char *buf, size_t len);
ARL2_API void arl2_profile_reset(void);

/*
 * Measure the bf16 matrix-core rate the current device sustains: one
 * launch of a pure MFMA loop (no memory traffic) with one 512-thread
 * workgroup per compute unit, each wavefront running `iters` rounds of four
 * independent 32x32x16 bf16 MFMA chains, timed with a pair of HIP events on
 * `stream` after one short warm-up launch. *tflops receives the flops
 * performed divided by the measured time, in TFLOP/s. It is the measured
 * counterpart of the published dense bf16 peak, against which a kernel's
 * fraction of peak is read. The call allocates and frees a small device
 * buffer and waits for the stream: not for use under graph capture.
 *   iters   rounds per wavefront, in [1, 2^20] (4096 gives about 0.5 ms on
 *           MI355X).
 *   tflops  host pointer, written on success only.
 * Errors: INVALID_ARG for a NULL tflops or iters out of range; ARL2_ERR_HIP
 * if the device query, the allocation, a launch or the events fail.
 */
ARL2_API arl2_status arl2_profile_mfma_peak(int32_t iters, double *tflops, void *stream);

/* Static text for a status code (never NULL). */
ARL2_API const char *arl2_status_string(int32_t status);

/* Detail of the last error returned on the calling thread ("" if none). */
ARL2_API const char *arl2_last_error(void);

/* ARL2_VERSION of the loaded library. */
ARL2_API int32_t arl2_version(void);

#ifdef __cplusplus
}
#endif
#endif /* ARL2_H */
