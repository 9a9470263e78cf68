"""Float64 CPU oracle of one ARL2 hybrid attention layer ("Attend Locally,
Remember Linearly").

TEST INFRASTRUCTURE ONLY. This module is the plain, slow, obviously correct
definition that the HIP library is checked against. Only the test suite, the
smoke check and the benchmark's CPU-baseline leg may import it; the library
itself never calls it and shares no code with it.

Every function below follows a passage of the pages that describe the method:

* [TS] "Technical Summary: Attend Locally, Remember Linearly (ARL2)"
  (gist.science), section 2.1 "Hybrid Attention Decomposition" and
  section 2.2 "Memory State Management";
* [NP] the NeurIPS 2026 poster abstract "Attend Locally, Remember Linearly:
  Linear Attention as Cross-Frame Memory for Autoregressive Video Diffusion";
* [AS] the atlas.scime.ai summary of the same paper, sections "Approach",
  "Surprising findings" and "Builds on" (Gated Delta Network).

Where the pages leave a step open this module takes the plainest reading and
says so in the function's docstring (softmax scale, no mask, row-vector
feature maps without bias, the L2 normalisation of Q' and K' with a 1e-6
floor, the transpose of K' in the update, the plain sum of the branches,
headwise-scalar alpha and per-token beta, and for the token-level ablation
the read of each token after its own write).

Arrays are float64; inputs that were stored in bfloat16 or float32 widen to
float64 exactly, so the oracle sees the same values as the GPU.
"""
from __future__ import annotations

import math
from typing import Tuple

import numpy as np

L2_EPS = 1e-6


# ------------------------------------------------------------ intra branch
def row_softmax(z: np.ndarray) -> np.ndarray:
    """Softmax over the last axis, shifted by the row maximum for stability."""
    m = np.max(z, axis=-1, keepdims=True)
    e = np.exp(z - m)
    return e / np.sum(e, axis=-1, keepdims=True)


def intra_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray) -> np.ndarray:
    """Intra-frame branch of [TS] section 2.1: full bidirectional softmax
    attention among the tokens of the current frame, for one head.

    q [Lq][d], k and v [Lk][d] -> [Lq][d]. No mask: every token attends to
    every token of the frame (bidirectional). The pages do not print the
    scale; the branch keeps the pretrained softmax attention, so it is the
    standard scaled dot product with scale 1/sqrt(d).

    The same definition with Lk > Lq is the full-softmax attention over a
    growing key/value cache that the method replaces ([TS] section 1).
    """
    d = q.shape[-1]
    z = (q @ k.T) / math.sqrt(d)
    return row_softmax(z) @ v


# ------------------------------------------------------------ inter branch
def feature_map(x: np.ndarray, W: np.ndarray) -> np.ndarray:
    """Per-head grouped 1x1 feature map of [TS] section 2.1 (phi_q, phi_k,
    phi_v): one d x d linear map per head applied to every token.

    Reading: row-vector convention x' = x W with W stored [d_in][d_out], no
    bias (the pages give neither an orientation nor a bias).
    """
    return x @ W


def l2_normalize_rows(x: np.ndarray, eps: float = L2_EPS) -> np.ndarray:
    """Scale every token's vector to unit Euclidean length.

    Not on the pages: this implementation's stated choice for Q' and K'.
    A row of norm below ``eps`` is divided by ``eps`` (a zero row stays zero).
    """
    n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True))
    return x / np.maximum(n, eps)


def inter_read(Qp: np.ndarray, S: np.ndarray) -> np.ndarray:
    """Inter-frame read of [TS] section 2.1: O_inter = Q'_N S_{N-1}.

    Qp [L][d_k], S [d_k][d_v] -> [L][d_v]. Every token of the frame reads the
    same pre-update state (frame-level access, [TS] section 2.2).
    """
    return Qp @ S


def gate_state(S: np.ndarray, alpha) -> np.ndarray:
    """The forget gate's action on the state.

    Headwise gating (the method's choice, [TS] section 4 and [AS]
    "Surprising findings"): alpha is one scalar per head and frame and
    scales the whole state. Elementwise gating (the ablation those passages
    compare against): the pages give no formula; the reading here is one
    gate per key channel, alpha [d_k], scaling row i of S (d_k x d_v) by
    alpha_i, i.e. diag(alpha) S.
    """
    a = np.asarray(alpha, dtype=np.float64)
    if a.ndim == 0:
        return float(a) * S
    assert a.shape == (S.shape[0],), "elementwise gate: one value per d_k row"
    return a[:, None] * S


def delta_update(S: np.ndarray, Kp: np.ndarray, Vp: np.ndarray, alpha,
                 beta: np.ndarray) -> np.ndarray:
    """Gated delta state update of [TS] section 2.1, one frame:

        R   = V' - K' S_{N-1}                     (residual of every token)
        S_N = gate(S_{N-1}) + K'^T diag(beta) R,  gate(S) = alpha S

    S [d_k][d_v], Kp [L][d_k], Vp [L][d_v], alpha a scalar (headwise gate of
    this frame; or [d_k] for elementwise gating, see gate_state), beta [L]
    (one learning rate per token). The printed formula omits the transpose;
    with tokens as rows of K' the product that yields a d_k x d_v matrix is
    K'^T (...). The gate acts on the carried state only; the residual reads
    the ungated S_{N-1}. Returns the new state (a new array).
    """
    R = Vp - Kp @ S
    return gate_state(S, alpha) + Kp.T @ (beta[:, None] * R)


def token_level_update(S: np.ndarray, Kp: np.ndarray, Vp: np.ndarray, alpha: float,
                       beta: np.ndarray) -> np.ndarray:
    """The token-level access that the pages' ablation compares against
    ([TS] section 4, [AS] "Surprising findings"): tokens of the frame write
    the state one after another, each applying the update of [TS] section 2.1
    with a single token,
        S_i = a_i S_{i-1} + beta_i k_i (v_i - k_i^T S_{i-1}),
    where the frame's forget gate is applied with the first token only
    (a_1 = alpha, a_i = 1 after it), so that a one-token frame gives the
    frame-level result. Used only to show that frame-level access differs
    from it.
    """
    for i in range(Kp.shape[0]):
        k = Kp[i]
        a = alpha if i == 0 else 1.0
        S = a * S + beta[i] * np.outer(k, Vp[i] - k @ S)
    return S


def token_level_head_forward(q: np.ndarray, k: np.ndarray, v: np.ndarray, Wq: np.ndarray,
                             Wk: np.ndarray, Wv: np.ndarray, S: np.ndarray, alpha: float,
                             beta: np.ndarray, update: bool) -> Tuple[np.ndarray, np.ndarray]:
    """One pass of one head with token-level access, the ablation that
    frame-level access is compared with ([TS] section 4, [AS] "Surprising
    findings"; [TS] section 2.2 describes the frame-level design it departs
    from).

    The pages name the ablation and report worse quality, nothing more. The
    reading here: inside the frame the tokens write the state one after
    another (``token_level_update``), and token i's query reads the state
    right after its own write, O_inter[i] = q'_i S_i, the order of the Gated
    Delta Network recurrence the method builds on ([AS] "Builds on"). The
    intra branch and the plain sum are unchanged. Clean-pass updates still
    hold: on a noisy pass the within-frame states only serve the reads and
    are dropped; on the clean pass S_L becomes S_N. alpha and beta are used
    on every pass. Returns (out, S_next).
    """
    o_intra = intra_attention(q, k, v)
    Qp = l2_normalize_rows(feature_map(q, Wq))
    Kp = l2_normalize_rows(feature_map(k, Wk))
    Vp = feature_map(v, Wv)
    o_inter = np.empty_like(o_intra)
    Si = S
    for i in range(Kp.shape[0]):
        a = alpha if i == 0 else 1.0
        Si = token_level_update(Si, Kp[i:i + 1], Vp[i:i + 1], a, beta[i:i + 1])
        o_inter[i] = Qp[i] @ Si
    return o_intra + o_inter, (Si if update else S)


def token_level_frame_forward(q: np.ndarray, k: np.ndarray, v: np.ndarray, Wphi: np.ndarray,
                              S: np.ndarray, alpha, beta, update_flag: int) -> np.ndarray:
    """``frame_forward`` with token-level access (``token_level_head_forward``
    per stream and head). alpha [B][H] and beta [B][L][H] are required on
    every pass. S [B][H][d][d] is updated in place on the clean pass."""
    assert update_flag in (0, 1)
    B, L, H, d = q.shape
    q, k, v = (np.asarray(t, dtype=np.float64) for t in (q, k, v))
    W = np.asarray(Wphi, dtype=np.float64)
    out = np.empty((B, L, H, d), dtype=np.float64)
    new_states = {}
    for b in range(B):
        for h in range(H):
            o, s_next = token_level_head_forward(
                q[b, :, h], k[b, :, h], v[b, :, h], W[0, h], W[1, h], W[2, h], S[b, h],
                float(alpha[b][h]), np.asarray(beta[b][:, h], dtype=np.float64),
                bool(update_flag))
            out[b, :, h] = o
            if update_flag:
                new_states[(b, h)] = s_next
    for (b, h), s_next in new_states.items():
        S[b, h] = s_next
    return out


# ------------------------------------------------------------ gates
def sigmoid(x: np.ndarray) -> np.ndarray:
    return 1.0 / (1.0 + np.exp(-x))


def gate_projections(x: np.ndarray, Wa: np.ndarray, Wb: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """The gates from the layer's token inputs ([TS] section 2.1: the gates
    are learned per-token projections; [TS] section 4 and [AS] "Surprising
    findings": the forget gate is headwise).

    x [B][L][D] (the tokens entering the layer), Wa, Wb [D][H] -> alpha [B][H],
    beta [B][L][H]. beta is one learning rate per token and head:
    sigmoid(x_i . Wb[:, h]). The pages do not say how the per-token
    projections become one forget gate per head and frame; the reading here
    is the plainest pooling, the mean over the frame's tokens of the logits:
    alpha[b][h] = sigmoid(mean_i x_i . Wa[:, h]). No bias.
    """
    x = np.asarray(x, dtype=np.float64)
    za = x @ np.asarray(Wa, dtype=np.float64)   # [B][L][H]
    zb = x @ np.asarray(Wb, dtype=np.float64)
    return sigmoid(za.mean(axis=1)), sigmoid(zb)


# ------------------------------------------------------------ one layer
def head_forward(q: np.ndarray, k: np.ndarray, v: np.ndarray, Wq: np.ndarray,
                 Wk: np.ndarray, Wv: np.ndarray, S: np.ndarray, alpha,
                 beta: np.ndarray, update: bool) -> Tuple[np.ndarray, np.ndarray]:
    """One pass of one head of one stream.

    out = O_intra + O_inter: the pages say the layer splits attention into the
    two branches but not how they are merged; the plain sum is this
    implementation's reading. O_inter reads the pre-update state; only a clean
    pass (``update``) produces S_N ([TS] section 2.2). Returns (out, S_next);
    S_next is S itself when no update happens.
    """
    o_intra = intra_attention(q, k, v)
    Qp = l2_normalize_rows(feature_map(q, Wq))
    out = o_intra + inter_read(Qp, S)
    if not update:
        return out, S
    Kp = l2_normalize_rows(feature_map(k, Wk))
    Vp = feature_map(v, Wv)
    return out, delta_update(S, Kp, Vp, alpha, beta)


def frame_forward(q: np.ndarray, k: np.ndarray, v: np.ndarray, Wphi: np.ndarray,
                  S: np.ndarray, alpha, beta, update_flag: int) -> np.ndarray:
    """One pass of the layer over a batch of streams.

    q, k, v [B][L][H][d] (token-major); Wphi [3][H][d][d] (maps for q, k, v);
    S [B][H][d][d] float64, updated IN PLACE when ``update_flag`` is 1 and
    left untouched when it is 0 ([TS] section 2.2: denoising passes only
    read, the clean pass writes); alpha [B][H] (headwise) or [B][H][d]
    (elementwise, see gate_state); beta [B][L][H].
    Returns out [B][L][H][d] float64.
    """
    assert update_flag in (0, 1)
    B, L, H, d = q.shape
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    W = np.asarray(Wphi, dtype=np.float64)
    out = np.empty((B, L, H, d), dtype=np.float64)
    new_states = {}
    for b in range(B):
        for h in range(H):
            a = np.asarray(alpha[b][h], dtype=np.float64) if update_flag else 0.0
            be = np.asarray(beta[b][:, h], dtype=np.float64) if update_flag else None
            o, s_next = head_forward(q[b, :, h], k[b, :, h], v[b, :, h], W[0, h], W[1, h],
                                     W[2, h], S[b, h], a, be, bool(update_flag))
            out[b, :, h] = o
            if update_flag:
                new_states[(b, h)] = s_next
    # Every head of the frame read the pre-update state above; write after.
    for (b, h), s_next in new_states.items():
        S[b, h] = s_next
    return out


def output_rows(q: np.ndarray, k: np.ndarray, v: np.ndarray, Wq: np.ndarray,
                S: np.ndarray, rows: np.ndarray) -> np.ndarray:
    """out for a subset of query rows of one head (the same definition as
    ``head_forward``, restricted to the requested rows; used to check large
    workloads on sampled outputs). q/k/v [L][d], S [d][d] pre-update."""
    qs = np.asarray(q, dtype=np.float64)[rows]
    o_intra = intra_attention(qs, np.asarray(k, np.float64), np.asarray(v, np.float64))
    Qp = l2_normalize_rows(feature_map(qs, np.asarray(Wq, np.float64)))
    return o_intra + inter_read(Qp, S)


def kv_cache_attention(q: np.ndarray, kc: np.ndarray, vc: np.ndarray) -> np.ndarray:
    """Full-softmax attention of one frame's queries over a key/value cache,
    per stream and head: q [B][Lq][H][d], kc/vc [B][Lk][H][d] -> [B][Lq][H][d].
    This is the attention whose growing cache the method removes ([TS]
    section 1); it is the same definition as ``intra_attention``."""
    B, Lq, H, d = q.shape
    out = np.empty((B, Lq, H, d), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            out[b, :, h] = intra_attention(np.asarray(q[b, :, h], np.float64),
                                           np.asarray(kc[b, :, h], np.float64),
                                           np.asarray(vc[b, :, h], np.float64))
    return out
