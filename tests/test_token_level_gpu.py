"""Token-level state access on the GPU vs the float64 oracle, through the C ABI.

Same bar as the frame-level parity tests: outputs within 2e-2 (bf16 io) /
1e-4 (fp32 io) max-norm relative error per (stream, head) and pass, state
within 1e-3 per (stream, head). Shapes cover one and several 64-token chunks,
a ragged last chunk, a single token, the full 480p frame and the token-by-
token kernel used for fp32 io and d = 16.
"""
import numpy as np
import pytest

import oracle as O
import synth_inputs as SI
from parity_utils import (TOL_OUT, TOL_S, device, out_err_per_head, state_err, to_dev,
                          to_host)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lay():
    import torch  # noqa: F401
    device()
    from hybrid_softmax_gated_amd import layer
    return layer


def _run(lay, w, frames=None):
    """Every pass of ``w`` with token-level access on the GPU and in the
    oracle; returns the per-pass output errors, the per-frame state errors
    and whether noisy passes left S bitwise unchanged."""
    import torch
    dtype = 0 if w.dtype == SI.BF16 else 1
    L = lay.ARL2Layer(w.B, w.H, w.d, w.L, dtype)
    W = SI.make_weights(w)
    Wd = to_dev(W, w.dtype)
    S_ref = SI.make_state0(w).astype(np.float64)
    if np.any(S_ref):
        L.reset(torch.from_numpy(S_ref.astype(np.float32)).to(device()))
    out = torch.empty((w.B, w.L, w.H, w.d), dtype=SI.torch_dtype(w.dtype), device=device())
    e_out, e_s, noisy_kept = [], [], True
    for p in SI.iter_passes(w, frames):
        q, k, v = (to_dev(x, w.dtype) for x in (p.q, p.k, p.v))
        al = torch.from_numpy(p.alpha).to(device())
        be = torch.from_numpy(p.beta).to(device())
        S_before = L.S.clone()
        L.forward_token_level(q, k, v, Wd, al, be, out, p.update)
        ref = O.token_level_frame_forward(p.q, p.k, p.v, W, S_ref, p.alpha, p.beta,
                                          int(p.update))
        torch.cuda.synchronize()
        e_out.append(out_err_per_head(to_host(out), ref))
        if p.update:
            e_s.append(state_err(to_host(L.S), S_ref))
        else:
            noisy_kept &= bool(torch.equal(L.S, S_before))
    return e_out, e_s, noisy_kept


@pytest.mark.parametrize("B,H,L,frames,noisy", [
    (1, 2, 200, 2, 1),     # three chunks and a ragged fourth, two frames
    (2, 3, 64, 1, 1),      # exactly one chunk, two streams
    (1, 1, 1, 2, 0),       # a single token per frame
    (1, 2, 130, 3, 1),     # two chunks and two tokens, three frames
])
def test_token_level_mfma_path(lay, B, H, L, frames, noisy):
    w = SI.Workload("tl", B, H, 128, L, frames, noisy, SI.BF16, 0.02, seed=L + 7 * B)
    e_out, e_s, kept = _run(lay, w)
    print(f"\n[token-level bf16] B={B} H={H} L={L}: out {max(e_out):.2e} S {max(e_s):.2e}",
          flush=True)
    assert max(e_out) <= TOL_OUT[SI.BF16]
    assert max(e_s) <= TOL_S
    assert kept


@pytest.mark.parametrize("Bn,H", [(1, 65535), (65535, 1)])
def test_token_level_maximum_heads_and_streams(lay, Bn, H):
    """Token-level access with the largest head and stream counts accepted
    (65,535), 64-token frames (one chunk record per (stream, head)): one
    noisy and one clean pass drawn on the GPU; the first, last and middle
    (stream, head) pairs are checked against the oracle."""
    import torch
    L, d = 64, 128
    dev = device()
    g = torch.Generator(device=dev)
    g.manual_seed(Bn * 11 + H)
    W = (torch.eye(d, device=dev) + 0.01 * torch.randn((3, H, d, d), generator=g, device=dev))
    W = W.to(torch.bfloat16)
    S0 = 0.02 * torch.randn((Bn, H, d, d), generator=g, device=dev)
    layer = lay.ARL2Layer(Bn, H, d, L, 0)
    layer.reset(S0)
    out = torch.empty((Bn, L, H, d), dtype=torch.bfloat16, device=dev)
    pairs = sorted({(0, 0), (Bn - 1, H - 1), (Bn // 2, H // 2), (Bn - 1, 0), (0, H - 1)})
    S_ref = {bh: S0[bh].double().cpu().numpy() for bh in pairs}
    for update in (0, 1):
        q, k, v = (torch.randn((Bn, L, H, d), generator=g, device=dev).to(torch.bfloat16)
                   for _ in range(3))
        alpha = torch.sigmoid(2 + 0.5 * torch.randn((Bn, H), generator=g, device=dev))
        beta = torch.sigmoid(torch.randn((Bn, L, H), generator=g, device=dev))
        layer.forward_token_level(q, k, v, W, alpha, beta, out, update)
        torch.cuda.synchronize()
        for b, h in pairs:
            def one(t):
                return t[b:b + 1, :, h:h + 1].float().cpu().numpy()
            Sh = S_ref[(b, h)][None, None].copy()
            ref = O.token_level_frame_forward(one(q), one(k), one(v),
                                              W[:, h:h + 1].float().cpu().numpy(), Sh,
                                              alpha[b:b + 1, h:h + 1].cpu().numpy(),
                                              beta[b:b + 1, :, h:h + 1].cpu().numpy(), update)
            err = np.max(np.abs(one(out) - ref)) / np.max(np.abs(ref))
            assert err <= TOL_OUT[SI.BF16], (b, h, update, err)
            if update:
                S_ref[(b, h)] = Sh[0, 0]
    for b, h in pairs:
        ref = S_ref[(b, h)]
        err = np.max(np.abs(layer.S[b, h].double().cpu().numpy() - ref)) / np.max(np.abs(ref))
        assert err <= TOL_S, (b, h, err)


def test_token_level_480p_frame(lay):
    """The 480p frame step (12 heads, 1560 tokens = 24 chunks + 24 tokens):
    one noisy and one clean pass from a warm state."""
    w = SI.WORKLOADS["frame_step_480p"]
    e_out, e_s, kept = _run(lay, w)
    print(f"\n[token-level 480p] out {max(e_out):.2e} S {max(e_s):.2e}", flush=True)
    assert max(e_out) <= TOL_OUT[SI.BF16]
    assert max(e_s) <= TOL_S
    assert kept


@pytest.mark.parametrize("dtype,d,B,H,L", [
    (SI.F32, 16, 2, 2, 50),
    (SI.F32, 128, 1, 2, 20),
    (SI.BF16, 16, 1, 3, 33),
])
def test_token_level_token_by_token_kernel(lay, dtype, d, B, H, L):
    w = SI.Workload("tlg", B, H, d, L, 2, 1, dtype, 0.02, seed=d + L)
    e_out, e_s, kept = _run(lay, w)
    print(f"\n[token-level {dtype} d={d}] out {max(e_out):.2e} S {max(e_s):.2e}", flush=True)
    assert max(e_out) <= TOL_OUT[dtype]
    assert max(e_s) <= TOL_S
    assert kept


def test_token_level_is_not_frame_level_and_is_repeatable(lay):
    """The two accesses give different states on the same inputs (the GPU
    agrees with the oracle on which), and token-level runs are bitwise
    reproducible."""
    import torch
    w = SI.Workload("tlr", 1, 2, 128, 150, 1, 0, SI.BF16, 0.02, seed=3)
    p = next(SI.iter_passes(w))
    W = SI.make_weights(w)
    S0 = torch.from_numpy(SI.make_state0(w)).to(device())
    q, k, v = (to_dev(x, w.dtype) for x in (p.q, p.k, p.v))
    al = torch.from_numpy(p.alpha).to(device())
    be = torch.from_numpy(p.beta).to(device())
    Wd = to_dev(W, w.dtype)
    res = []
    for mode in ("token", "token", "frame"):
        L = lay.ARL2Layer(w.B, w.H, w.d, w.L, 0)
        L.reset(S0)
        out = torch.empty((w.B, w.L, w.H, w.d), dtype=torch.bfloat16, device=device())
        if mode == "token":
            L.forward_token_level(q, k, v, Wd, al, be, out, True)
        else:
            L.forward(q, k, v, Wd, al, be, out, True)
        torch.cuda.synchronize()
        res.append((out.clone(), L.S.clone()))
    assert torch.equal(res[0][0], res[1][0]) and torch.equal(res[0][1], res[1][1])
    d_gpu = (res[0][1] - res[2][1]).abs().max().item()
    S_t = SI.make_state0(w).astype(np.float64)
    S_f = S_t.copy()
    O.token_level_frame_forward(p.q, p.k, p.v, W, S_t, p.alpha, p.beta, 1)
    O.frame_forward(p.q, p.k, p.v, W, S_f, p.alpha, p.beta, 1)
    d_ref = np.abs(S_t - S_f).max()
    assert d_ref > 1e-2 and abs(d_gpu - d_ref) <= 1e-3 * np.abs(S_t).max() + 1e-3 * d_ref
