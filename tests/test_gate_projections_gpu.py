"""Gate projections on the GPU vs the float64 oracle, through the C ABI.

Tolerance, from the arithmetic: both paths see the same io-dtype values.
The GPU sums the D products of a logit in fp32 in some order, so its error is
at most gamma_n * sum_i |x_i w_i| with gamma_n = n u / (1 - n u), u = 2^-24
and n the number of additions (D for beta; D + L for the alpha logit, whose
mean also sums over the L tokens). The logistic function has slope at most
1/4, and its fp32 evaluation adds a few units in the last place; 2e-6
covers that.
"""
import numpy as np
import pytest

import oracle as O
import synth_inputs as SI
from parity_utils import device, to_dev

pytestmark = pytest.mark.gpu

U = 2.0 ** -24


def _gamma(n):
    return n * U / (1 - n * U)


def _oracle_and_bounds(x, Wa, Wb):
    x64, a64, b64 = (np.asarray(t, np.float64) for t in (x, Wa, Wb))
    alpha, beta = O.gate_projections(x64, a64.T, b64.T)
    L, D = x.shape[1], x.shape[2]
    tol_b = 0.25 * _gamma(D) * (np.abs(x64) @ np.abs(b64).T) + 2e-6           # [B][L][H]
    tol_a = 0.25 * _gamma(D + L) * (np.abs(x64) @ np.abs(a64).T).mean(axis=1) + 2e-6  # [B][H]
    return alpha, beta, tol_a, tol_b


@pytest.fixture(scope="module")
def lay():
    import torch  # noqa: F401
    device()
    from hybrid_softmax_gated_amd import layer
    return layer


def _run(lay, B, L, D, H, dtype, seed):
    import torch
    x, Wa, Wb = SI.make_gate_inputs(B, L, D, H, dtype, seed)
    dt = 0 if dtype == SI.BF16 else 1
    alpha, beta, _ = lay.gate_projections(to_dev(x, dtype), to_dev(Wa, dtype), to_dev(Wb, dtype),
                                          dt)
    torch.cuda.synchronize()
    a_ref, b_ref, tol_a, tol_b = _oracle_and_bounds(x, Wa, Wb)
    ga = alpha.cpu().numpy().astype(np.float64)
    gb = beta.cpu().numpy().astype(np.float64)
    return ga, gb, a_ref, b_ref, tol_a, tol_b


@pytest.mark.parametrize("B,L,D,H,dtype", [
    (1, 1560, 1536, 12, SI.BF16),   # 480p frame: 30x52 tokens, width 1536, 12 heads
    (2, 200, 1536, 12, SI.BF16),    # ragged token tile, two streams
    (1, 77, 192, 20, SI.BF16),      # two column tiles (40 gate columns), three groups of D
    (3, 1, 64, 1, SI.BF16),         # one token: alpha is that token's gate
    (1, 130, 100, 5, SI.BF16),      # D not a multiple of 64: generic kernel
    (2, 50, 48, 3, SI.F32),         # fp32 io
    (1, 3600, 1536, 12, SI.BF16),   # 720p frame: 45x80 tokens
    (1, 37, 1 << 16, 3, SI.BF16),   # the widest input accepted (D = 2^16)
])
def test_gate_projections_match_oracle(lay, B, L, D, H, dtype):
    ga, gb, a_ref, b_ref, tol_a, tol_b = _run(lay, B, L, D, H, dtype, seed=B * 1000 + L)
    print(f"\n[gate] B={B} L={L} D={D} H={H} {dtype}: |da| {np.max(np.abs(ga - a_ref)):.2e} "
          f"|db| {np.max(np.abs(gb - b_ref)):.2e}", flush=True)
    assert np.all(np.abs(ga - a_ref) <= tol_a)
    assert np.all(np.abs(gb - b_ref) <= tol_b)
    # the gates are not degenerate on these inputs
    assert np.ptp(gb) > 0.3 and np.all((ga > 0) & (ga < 1))


def test_gate_projections_repeatable(lay):
    import torch
    x, Wa, Wb = SI.make_gate_inputs(1, 1560, 1536, 12, SI.BF16, 5)
    xd, ad, bd = (to_dev(t, SI.BF16) for t in (x, Wa, Wb))
    a1, b1, ws = lay.gate_projections(xd, ad, bd, 0)
    ws.fill_(255)   # the workspace needs no initialisation
    a2, b2, _ = lay.gate_projections(xd, ad, bd, 0, ws=ws)
    torch.cuda.synchronize()
    assert torch.equal(a1, a2) and torch.equal(b1, b2)


def test_gates_feed_the_frame_step(lay):
    """Gates from the projections drive a clean pass; the state matches the
    oracle run on the oracle's own gates."""
    import torch
    from parity_utils import oracle_state_update, state_err, to_host
    B, L, H, d, D = 1, 300, 12, 128, 1536
    x, Wa, Wb = SI.make_gate_inputs(B, L, D, H, SI.BF16, 9)
    alpha, beta, _ = lay.gate_projections(to_dev(x, SI.BF16), to_dev(Wa, SI.BF16),
                                          to_dev(Wb, SI.BF16), 0)
    a_ref, b_ref = O.gate_projections(x.astype(np.float64), Wa.T.astype(np.float64),
                                      Wb.T.astype(np.float64))
    p = SI.random_pass(B, H, d, L, SI.BF16, seed=9)
    w = SI.Workload("gates", B, H, d, L, 1, 0, SI.BF16, 0.02, 9)
    W = SI.make_weights(w)
    S0 = SI.make_state0(w)
    layer = lay.ARL2Layer(B, H, d, L, 0)
    layer.reset(torch.from_numpy(S0).to(device()))
    out = torch.empty((B, L, H, d), dtype=torch.bfloat16, device=device())
    q, k, v = (to_dev(t, SI.BF16) for t in (p.q, p.k, p.v))
    layer.forward(q, k, v, to_dev(W, SI.BF16), alpha, beta, out, True)
    torch.cuda.synchronize()
    S_ref = S0.astype(np.float64)
    oracle_state_update(S_ref, p.k, p.v, W, a_ref, b_ref)
    err = state_err(to_host(layer.S), S_ref)
    print(f"\n[gate->frame] state err {err:.2e}", flush=True)
    assert err < 1e-3
