"""Seeded synthetic inputs for the ARL2 hybrid attention layer.

This module is shared by the float64 oracle (``oracle/``) and the HIP path
(``hybrid_softmax_gated_amd``). It draws random numbers and rounds them to the
storage type; it holds none of the layer's arithmetic, so both sides consume
identical bytes without sharing any computation.

Workload recipe (the pages give the model shape, not the activations):

* q, k, v ~ N(0, 1) per element, fresh for every pass (noisy and clean), in
  token-major layout [B][L][H][d].
* phi weights W = I + N(0, 0.01) (the second argument is a standard
  deviation), one d x d map per (map in {q, k, v}, head), layout [3][H][d][d],
  drawn once per run and shared by every stream of a batch.
* alpha = sigmoid(N(2, 0.5)) per (stream, head, frame) (per (stream, head,
  frame, d_k row) for elementwise gating), beta = sigmoid(N(0, 1)) per
  (stream, token, head, frame), fp32.
* S0 = 0, or N(0, 0.02) per element where a workload asks for a warm state.
* Gate projections (``make_gate_inputs``): layer input x [B][L][D] =
  mu_b + N(0, 1) per element with a per-stream channel mean mu_b ~ N(0, 0.5),
  so that the frame-pooled logits are not all near zero; weights Wa, Wb
  [H][D] ~ N(0, 1/D), so the logits are of order one.
* For bf16 workloads every io tensor (q, k, v, W) is drawn in float32 and
  rounded to bfloat16 with round-to-nearest-even; the float32 arrays returned
  here hold exactly the bf16 values, and ``bits`` arrays hold the raw bf16
  patterns that are uploaded to the GPU.

Generators: ``numpy.random.default_rng`` (PCG64), one per purpose, seeded with
``[tag, seed]`` so that weights, state and per-stream activations are
independent streams whose draws do not depend on each other's sizes.
"""
from __future__ import annotations

import dataclasses
from typing import Iterator, List, Optional

import numpy as np

BF16 = "bf16"
F32 = "f32"

_TAG_W = 11
_TAG_S0 = 12
_TAG_STREAM = 13
_TAG_GATE = 14


# ---------------------------------------------------------------- bf16 bytes
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even).

    Returns the 16-bit patterns as uint16. NaN inputs stay NaN (quiet bit set).
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    nan = np.isnan(x)
    # For every non-NaN pattern the sum stays below 2**32.
    r = u + (np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))
    out = (r >> np.uint32(16)).astype(np.uint16)
    if nan.any():
        out = np.where(nan, ((u >> np.uint32(16)) | np.uint32(0x40)).astype(np.uint16), out)
    return out


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bfloat16 patterns (uint16) to the float32 values they encode (exact)."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    out = np.empty(b.shape, dtype=np.uint32)
    np.left_shift(b, 16, out=out, dtype=np.uint32)
    return out.view(np.float32)


def round_f32_to_bf16_values(x: np.ndarray) -> np.ndarray:
    """float32 array holding the bf16-rounded values of ``x``."""
    return bf16_bits_to_f32(f32_to_bf16_bits(x))


def _sigmoid(x: np.ndarray) -> np.ndarray:
    # Gate values are inputs to the layer, drawn as the logistic function of a
    # normal sample; this is part of the input recipe, not of the layer.
    return (1.0 / (1.0 + np.exp(-x.astype(np.float64)))).astype(np.float32)


# ------------------------------------------------------------------ configs
@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic workload: shapes, pass schedule and input distributions."""

    name: str
    B: int
    H: int
    d: int
    L: int
    frames: int
    noisy_passes: int      # query-only passes per frame before the clean pass
    dtype: str             # io dtype of q, k, v, W, out: "bf16" or "f32"
    s0_std: float          # 0 => S0 = 0
    seed: int = 0          # stream b uses seed + b
    beta_scale: float = 1.0  # companion runs multiply beta by 1/L
    w_std: float = 0.01
    gate: str = "headwise"   # "elementwise": alpha has one value per d_k row

    @property
    def passes_per_frame(self) -> int:
        return self.noisy_passes + 1


# The five workloads: the tiny fp32 exactness case, one Wan2.1-1.3B frame step
# at 480p (30x52 latent tokens after 2x2 patchify, 12 heads of 128), the
# 21-latent-frame stream with 4 noisy + 1 clean pass, the 231-frame long
# horizon, and the batched 720p case (45x80 tokens, 4 streams).
WORKLOADS = {
    "tiny_f32": Workload("tiny_f32", 1, 1, 16, 64, 8, 0, F32, 0.0),
    "frame_step_480p": Workload("frame_step_480p", 1, 12, 128, 1560, 1, 1, BF16, 0.02),
    "stream21_480p": Workload("stream21_480p", 1, 12, 128, 1560, 21, 4, BF16, 0.0),
    "long231_480p": Workload("long231_480p", 1, 12, 128, 1560, 231, 1, BF16, 0.02),
    "batched720p": Workload("batched720p", 4, 12, 128, 3600, 21, 4, BF16, 0.0),
}


def companion(w: Workload) -> Workload:
    """The same workload with beta divided by L (keeps the state bounded)."""
    return dataclasses.replace(w, name=w.name + "_beta_over_L", beta_scale=1.0 / w.L)


def scaled(w: Workload, **kw) -> Workload:
    """A copy of ``w`` with some fields replaced (smaller shapes for tests)."""
    return dataclasses.replace(w, **kw)


# ------------------------------------------------------------------ drawing
@dataclasses.dataclass
class PassInputs:
    """One pass of one frame: q, k, v in [B][L][H][d] (float32 values)."""

    frame: int
    index: int             # pass index within the frame; the last one is clean
    update: bool           # True for the clean pass
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    alpha: np.ndarray      # [B][H] (headwise) or [B][H][d] (elementwise) float32
    beta: np.ndarray       # [B][L][H] float32 (this frame's)
    dtype: str

    def bits(self, name: str) -> np.ndarray:
        """Raw bf16 patterns of q/k/v (bf16 workloads only)."""
        assert self.dtype == BF16
        return f32_to_bf16_bits(getattr(self, name))


def _store(x: np.ndarray, dtype: str) -> np.ndarray:
    x = x.astype(np.float32)
    return round_f32_to_bf16_values(x) if dtype == BF16 else x


def make_weights(w: Workload) -> np.ndarray:
    """phi weights [3][H][d][d] = I + N(0, w_std), io-dtype values as float32."""
    rng = np.random.default_rng([_TAG_W, w.seed])
    eye = np.eye(w.d, dtype=np.float32)
    W = eye[None, None] + rng.standard_normal((3, w.H, w.d, w.d), dtype=np.float32) * np.float32(w.w_std)
    return _store(W, w.dtype)


def make_state0(w: Workload) -> np.ndarray:
    """Initial state [B][H][d][d] float32 (zeros or N(0, s0_std))."""
    S = np.zeros((w.B, w.H, w.d, w.d), dtype=np.float32)
    if w.s0_std > 0:
        for b in range(w.B):
            rng = np.random.default_rng([_TAG_S0, w.seed + b])
            S[b] = rng.standard_normal((w.H, w.d, w.d), dtype=np.float32) * np.float32(w.s0_std)
    return S


def iter_passes(w: Workload, frames: Optional[int] = None) -> Iterator[PassInputs]:
    """Yield every pass of every frame in order.

    Per stream b the draw order is: for each frame, for each pass, q then k
    then v ([L][H][d] each); then alpha [H] and beta [L][H] of that frame.
    """
    nf = w.frames if frames is None else frames
    rngs = [np.random.default_rng([_TAG_STREAM, w.seed + b]) for b in range(w.B)]
    shape = (w.L, w.H, w.d)
    for f in range(nf):
        per_pass: List[List[np.ndarray]] = []
        for p in range(w.passes_per_frame):
            qkv = []
            for _name in ("q", "k", "v"):
                x = np.stack([r.standard_normal(shape, dtype=np.float32) for r in rngs])
                qkv.append(_store(x, w.dtype))
            per_pass.append(qkv)
        ashape = (w.H, w.d) if w.gate == "elementwise" else (w.H,)
        alpha = np.stack([_sigmoid(2.0 + 0.5 * r.standard_normal(ashape, dtype=np.float32))
                          for r in rngs])
        beta = np.stack([_sigmoid(r.standard_normal((w.L, w.H), dtype=np.float32)) for r in rngs])
        if w.beta_scale != 1.0:
            beta = (beta * np.float32(w.beta_scale)).astype(np.float32)
        for p, (q, k, v) in enumerate(per_pass):
            yield PassInputs(f, p, p == w.passes_per_frame - 1, q, k, v,
                             alpha.astype(np.float32), beta.astype(np.float32), w.dtype)


def random_pass(B: int, H: int, d: int, L: int, dtype: str, seed: int,
                update: bool = True) -> PassInputs:
    """A single pass with arbitrary shapes (tests of ragged and edge sizes)."""
    w = Workload("adhoc", B, H, d, L, 1, 0, dtype, 0.0, seed)
    pi = next(iter_passes(w))
    pi.update = update
    return pi


def make_gate_inputs(B: int, L: int, D: int, H: int, dtype: str, seed: int):
    """(x [B][L][D], Wa [H][D], Wb [H][D]) as io-dtype values in float32."""
    rng = np.random.default_rng([_TAG_GATE, seed])
    mu = rng.standard_normal((B, 1, D), dtype=np.float32) * np.float32(0.5)
    x = mu + rng.standard_normal((B, L, D), dtype=np.float32)
    sd = np.float32(1.0 / np.sqrt(D))
    Wa = rng.standard_normal((H, D), dtype=np.float32) * sd
    Wb = rng.standard_normal((H, D), dtype=np.float32) * sd
    return _store(x, dtype), _store(Wa, dtype), _store(Wb, dtype)


# ------------------------------------------------------- device-side drawing
@dataclasses.dataclass
class DevicePass:
    """One pass drawn on a torch device: q, k, v [B][L][H][d] in the io dtype,
    alpha [B][H] and beta [B][L][H] float32."""

    frame: int
    index: int
    update: bool
    q: "object"
    k: "object"
    v: "object"
    alpha: "object"
    beta: "object"


def torch_dtype(dtype: str):
    import torch
    return torch.bfloat16 if dtype == BF16 else torch.float32


def iter_passes_device(w: Workload, device, frames: Optional[int] = None) -> Iterator[DevicePass]:
    """The same recipe as ``iter_passes``, drawn with torch's seeded generator
    on ``device`` (Philox on a GPU), for streams too long to draw on the host.

    Per stream b (generator seeded with 1_000_003 * (seed + b) + 13) the draw
    order is: for each frame, alpha [H] and beta [L][H] of the frame, then for
    each pass q, k, v ([L][H][d] each, float32, then rounded to the io dtype
    with round-to-nearest-even). Consumers that need host copies (the oracle)
    copy these exact tensors back, so both sides read the same bytes.
    """
    import torch
    nf = w.frames if frames is None else frames
    gens = []
    for b in range(w.B):
        g = torch.Generator(device=device)
        g.manual_seed(1_000_003 * (w.seed + b) + _TAG_STREAM)
        gens.append(g)
    io = torch_dtype(w.dtype)
    shape = (w.L, w.H, w.d)
    for f in range(nf):
        ashape = (w.H, w.d) if w.gate == "elementwise" else (w.H,)
        alpha = torch.empty((w.B,) + ashape, dtype=torch.float32, device=device)
        beta = torch.empty((w.B, w.L, w.H), dtype=torch.float32, device=device)
        for b, g in enumerate(gens):
            alpha[b] = torch.sigmoid(2.0 + 0.5 * torch.randn(ashape, generator=g, device=device))
            beta[b] = torch.sigmoid(torch.randn((w.L, w.H), generator=g, device=device))
        if w.beta_scale != 1.0:
            beta *= w.beta_scale
        for p in range(w.passes_per_frame):
            t = []
            for _name in ("q", "k", "v"):
                x = torch.empty((w.B,) + shape, dtype=io, device=device)
                for b, g in enumerate(gens):
                    x[b] = torch.randn(shape, generator=g, device=device).to(io)
                t.append(x)
            yield DevicePass(f, p, p == w.passes_per_frame - 1, t[0], t[1], t[2], alpha, beta)
