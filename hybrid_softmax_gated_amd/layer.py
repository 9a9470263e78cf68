"""Device buffers for one ARL2 layer, allocated by torch, driven through the
C ABI. Torch is used for memory and streams only; every step of the layer
runs in libarl2's kernels."""
from __future__ import annotations

import torch

from . import binding as B

TORCH_DTYPE = {B.ARL2_BF16: torch.bfloat16, B.ARL2_F32: torch.float32}


class ARL2Layer:
    """State S [B][H][d][d] fp32 plus the workspace of one layer."""

    def __init__(self, Bn: int, H: int, d: int, L: int, dtype: int, device="cuda", stream=None):
        self.shape = (Bn, H, d, L)
        self.dtype = dtype
        self.S = torch.empty((Bn, H, d, d), dtype=torch.float32, device=device)
        self.ws_bytes = B.arl2_workspace_bytes(Bn, H, d, L, dtype)
        if self.ws_bytes == 0:
            raise ValueError(f"invalid layer shape {self.shape}")
        self.ws = torch.empty(self.ws_bytes, dtype=torch.uint8, device=device)
        self.st = B.arl2_state()
        B.arl2_state_init(self.st, Bn, H, d, L, dtype, self.S, self.ws, self.ws_bytes, stream)

    def reset(self, S0=None, stream=None) -> None:
        B.arl2_state_reset(self.st, S0, stream)

    def forward(self, q, k, v, W, alpha, beta, out, update: bool, stream=None,
                gate: str = "headwise") -> None:
        """One pass; gate "elementwise" takes alpha [B][H][d] (one gate per
        d_k row) instead of [B][H]."""
        if gate == "headwise":
            B.arl2_frame_forward(q, k, v, W, self.st, alpha, beta, out, 1 if update else 0, stream)
        else:
            B.arl2_frame_forward_gated(q, k, v, W, self.st, alpha, B.ARL2_GATE_ELEMENTWISE, beta,
                                       out, 1 if update else 0, stream)

    def forward_token_level(self, q, k, v, W, alpha, beta, out, update: bool,
                            stream=None) -> None:
        """One pass with token-level access: each token writes S in turn and
        reads it after its own write. The extra workspace is allocated once."""
        Bn, H, d, L = self.shape
        nb = B.arl2_token_level_workspace_bytes(Bn, H, d, L, self.dtype)
        if nb and (getattr(self, "tl_ws", None) is None or self.tl_ws.numel() < nb):
            self.tl_ws = torch.empty(nb, dtype=torch.uint8, device=self.S.device)
        B.arl2_frame_forward_token_level(q, k, v, W, self.st, alpha, beta, out,
                                         1 if update else 0, self.tl_ws if nb else None, nb,
                                         stream)


def softmax_attention(q, kc, vc, out, dtype: int, ws=None, stream=None):
    """Full-softmax attention over a key/value cache (the comparator);
    allocates the workspace with torch when none is given."""
    Bn, Lq, H, d = q.shape
    Lk = kc.shape[1]
    nb = B.arl2_softmax_attention_workspace_bytes(Bn, H, d, Lq, Lk, dtype)
    if ws is None or ws.numel() < nb:
        ws = torch.empty(nb, dtype=torch.uint8, device=q.device)
    B.arl2_softmax_attention(q, kc, vc, Bn, H, d, Lq, Lk, dtype, out, ws, nb, stream)
    return ws


def gate_projections(x, Wa, Wb, dtype: int, alpha=None, beta=None, ws=None, stream=None):
    """alpha [B][H] and beta [B][L][H] (fp32) from the layer input x [B][L][D]
    and the gate weights Wa, Wb [H][D]; allocates what is not given with
    torch. Returns (alpha, beta, ws)."""
    Bn, L, D = x.shape
    H = Wa.shape[0]
    nb = B.arl2_gate_projections_workspace_bytes(Bn, L, D, H, dtype)
    if nb == 0:
        raise ValueError(f"invalid gate projection shape B={Bn} L={L} D={D} H={H}")
    if ws is None or ws.numel() < nb:
        ws = torch.empty(nb, dtype=torch.uint8, device=x.device)
    if alpha is None:
        alpha = torch.empty((Bn, H), dtype=torch.float32, device=x.device)
    if beta is None:
        beta = torch.empty((Bn, L, H), dtype=torch.float32, device=x.device)
    B.arl2_gate_projections(x, Wa, Wb, Bn, L, D, H, dtype, alpha, beta, ws, nb, stream)
    return alpha, beta, ws
