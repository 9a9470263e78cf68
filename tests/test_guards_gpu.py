"""Guard bytes around every buffer of the 480p frame step.

q, k, v, the feature maps, alpha, beta, the state S, the workspace and out
are carved out of one device allocation, each followed by a gap of guard
bytes. After the query-only pass and after the clean pass (which writes S in
place) every guard byte must still hold its pattern, the read-only inputs
must be bitwise unchanged, the query-only pass must leave S bitwise
unchanged, and the results must match the float64 oracle. The pages put the
one in-place write of the method after the clean pass ("Technical Summary:
Attend Locally, Remember Linearly (ARL2)", section 2.2); this checks that
no kernel writes outside the buffers it was given.
"""
import numpy as np
import pytest

import oracle as O
import synth_inputs as SI
from parity_utils import TOL_OUT, TOL_S, device, rel_max_err, state_err, to_host

pytestmark = pytest.mark.gpu

GUARD = 4096
PATTERN = 0xA5


def _align(x, a=256):
    return (x + a - 1) // a * a


def test_guard_bytes_around_every_buffer_480p():
    import torch
    from hybrid_softmax_gated_amd import binding as Bd

    dev = device()
    w = SI.WORKLOADS["frame_step_480p"]
    B, H, d, L = w.B, w.H, w.d, w.L
    act = B * L * H * d * 2
    ws_bytes = Bd.arl2_workspace_bytes(B, H, d, L, Bd.ARL2_BF16)
    regions = [("q", act), ("k", act), ("v", act), ("W", 3 * H * d * d * 2),
               ("alpha", B * H * 4), ("beta", B * L * H * 4), ("S", B * H * d * d * 4),
               ("ws", ws_bytes), ("out", act)]
    offs, pos = {}, GUARD
    for name, n in regions:
        offs[name] = pos
        pos = _align(pos + n) + GUARD
    total = pos
    buf = torch.full((total,), PATTERN, dtype=torch.uint8, device=dev)
    guard = np.ones(total, dtype=bool)
    for name, n in regions:
        guard[offs[name]:offs[name] + n] = False
    sizes = dict(regions)

    def view(name, dtype, shape):
        return buf[offs[name]:offs[name] + sizes[name]].view(dtype).view(shape)

    q, k, v, out = (view(n, torch.bfloat16, (B, L, H, d)) for n in ("q", "k", "v", "out"))
    Wv = view("W", torch.bfloat16, (3, H, d, d))
    alpha = view("alpha", torch.float32, (B, H))
    beta = view("beta", torch.float32, (B, L, H))
    S = view("S", torch.float32, (B, H, d, d))
    ws = view("ws", torch.uint8, (ws_bytes,))

    W = SI.make_weights(w)
    Wv.copy_(torch.from_numpy(W).to(torch.bfloat16))
    S_ref = SI.make_state0(w).astype(np.float64)
    st = Bd.arl2_state()
    Bd.arl2_state_init(st, B, H, d, L, Bd.ARL2_BF16, S, ws, ws_bytes, None)
    S0 = torch.from_numpy(S_ref.astype(np.float32)).to(dev)
    Bd.arl2_state_reset(st, S0, None)

    def check_guards(when):
        host = buf.cpu().numpy()
        bad = np.flatnonzero(host[guard] != PATTERN)
        assert bad.size == 0, f"{bad.size} guard bytes changed {when}"

    check_guards("after init and reset")
    for p in SI.iter_passes(w):
        q.copy_(torch.from_numpy(p.q).to(torch.bfloat16))
        k.copy_(torch.from_numpy(p.k).to(torch.bfloat16))
        v.copy_(torch.from_numpy(p.v).to(torch.bfloat16))
        alpha.copy_(torch.from_numpy(p.alpha))
        beta.copy_(torch.from_numpy(p.beta))
        inputs = {n: buf[offs[n]:offs[n] + sizes[n]].clone()
                  for n in ("q", "k", "v", "W", "alpha", "beta")}
        S_before = S.clone()
        Bd.arl2_frame_forward(q, k, v, Wv, st, alpha, beta, out, int(p.update), None)
        torch.cuda.synchronize()
        when = "after the clean pass" if p.update else "after the query-only pass"
        check_guards(when)
        for n, t in inputs.items():
            assert torch.equal(buf[offs[n]:offs[n] + sizes[n]], t), f"{n} changed {when}"
        if not p.update:
            assert torch.equal(S, S_before), "the query-only pass changed S"
        ref = O.frame_forward(p.q, p.k, p.v, W, S_ref, p.alpha, p.beta, int(p.update))
        err = rel_max_err(to_host(out), ref)
        assert err < TOL_OUT[SI.BF16], (when, err)
        if p.update:
            assert state_err(to_host(S), S_ref) < TOL_S
