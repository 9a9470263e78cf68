"""An attention-only stack that mixes this layer with full-softmax layers.

The pages replace a share of a video DiT's self-attention layers by the
hybrid layer and keep the others as softmax attention over a key/value cache
of all earlier frames ("Technical Summary: Attend Locally, Remember Linearly
(ARL2)", section 4: three quarters of the layers replaced; section 1: the
cache that grows with every frame). This module holds the bookkeeping of
such a stack and nothing of its arithmetic: every layer's work runs in
libarl2's kernels (arl2_frame_forward for the hybrid layers,
arl2_softmax_attention for the cached ones). Torch provides the device
memory.

Cache rule of a softmax layer: within frame f every pass attends over the
cached keys/values of frames 0 .. f-1 followed by its own; the pass's own
keys/values are written into frame f's slot, so the slot ends up holding the
last (clean) pass's and becomes part of the cache for the frames after f.
The cache buffer grows by doubling its capacity in frames (copying what it
holds), so device memory grows with the frame index while copies stay
amortised.
"""
from __future__ import annotations

from typing import List, Optional

import torch

from . import binding as B
from .layer import ARL2Layer


class KVCache:
    """Keys and values of one softmax layer, [Bn][capacity * L][H][d]."""

    def __init__(self, Bn: int, L: int, H: int, d: int, dtype, device, capacity_frames: int = 1):
        self.Bn, self.L, self.H, self.d = Bn, L, H, d
        self.capacity = max(1, capacity_frames)
        self.k = torch.empty((Bn, self.capacity * L, H, d), dtype=dtype, device=device)
        self.v = torch.empty_like(self.k)
        self.frames = 0  # frames whose keys/values are held (slots 0 .. frames-1)

    def reserve(self, frames: int) -> None:
        """Make room for `frames` frames, keeping the frames held so far."""
        if frames <= self.capacity:
            return
        cap = self.capacity
        while cap < frames:
            cap *= 2
        k2 = torch.empty((self.Bn, cap * self.L, self.H, self.d), dtype=self.k.dtype,
                         device=self.k.device)
        v2 = torch.empty_like(k2)
        n = self.frames * self.L
        if n:
            k2[:, :n] = self.k[:, :n]
            v2[:, :n] = self.v[:, :n]
        self.k, self.v, self.capacity = k2, v2, cap

    def write(self, frame: int, k, v) -> None:
        """Store one pass's keys/values [Bn][L][H][d] in frame `frame`'s slot
        (frames are written in order; a later pass of the same frame
        overwrites the slot)."""
        if frame > self.frames or frame < self.frames - 1:
            raise ValueError(f"frame {frame} written out of order (cache holds {self.frames})")
        self.reserve(frame + 1)
        s = frame * self.L
        self.k[:, s:s + self.L] = k
        self.v[:, s:s + self.L] = v
        self.frames = frame + 1

    def keys(self, b: int):
        """Stream b's cached keys, [1][frames * L][H][d] (contiguous)."""
        return self.k[b:b + 1, :self.frames * self.L]

    def values(self, b: int):
        return self.v[b:b + 1, :self.frames * self.L]


class AttentionStack:
    """`layers` attention layers of one shape, the first `n_hybrid` of them
    this layer (state + workspace each) and the rest softmax attention over
    a key/value cache each."""

    def __init__(self, Bn: int, H: int, d: int, L: int, layers: int, n_hybrid: int,
                 dtype: int = B.ARL2_BF16, device="cuda"):
        if not 0 <= n_hybrid <= layers:
            raise ValueError(f"{n_hybrid} hybrid layers out of {layers}")
        self.shape = (Bn, H, d, L)
        self.dtype = dtype
        self.layers = layers
        self.n_hybrid = n_hybrid
        tdt = torch.bfloat16 if dtype == B.ARL2_BF16 else torch.float32
        self.hybrid: List[ARL2Layer] = [ARL2Layer(Bn, H, d, L, dtype, device)
                                        for _ in range(n_hybrid)]
        self.caches: List[KVCache] = [KVCache(Bn, L, H, d, tdt, device)
                                      for _ in range(layers - n_hybrid)]
        self.ws: Optional[torch.Tensor] = None
        self.device = device

    def kind(self, li: int) -> str:
        return "hybrid" if li < self.n_hybrid else "softmax"

    def forward(self, li: int, frame: int, q, k, v, W, alpha, beta, out, update: bool,
                stream=None) -> None:
        """One pass of layer `li` on frame `frame`. W, alpha, beta and update
        are used by hybrid layers only."""
        if li < self.n_hybrid:
            self.hybrid[li].forward(q, k, v, W, alpha, beta, out, update, stream)
            return
        cache = self.caches[li - self.n_hybrid]
        cache.write(frame, k, v)
        Bn, H, d, L = self.shape
        Lk = cache.frames * L
        nb = B.arl2_softmax_attention_workspace_bytes(1, H, d, L, Lk, self.dtype)
        if self.ws is None or self.ws.numel() < nb:
            self.ws = torch.empty(nb, dtype=torch.uint8, device=self.device)
        for b in range(Bn):
            B.arl2_softmax_attention(q[b:b + 1], cache.keys(b), cache.values(b), 1, H, d, L, Lk,
                                     self.dtype, out[b:b + 1], self.ws, self.ws.numel(), stream)
