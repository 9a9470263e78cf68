"""The frame step captured into a HIP graph gives, replay after replay, the
same bytes as the same calls made eagerly.

Every entry point on the frame step's path launches kernels only (the state
is cleared by a kernel, not a memset), so a caller may capture a pass, or a
whole frame, and replay it. Each replay here is checked bitwise against an
eager run of the same calls on a second state that follows the same
sequence, with eager work and synchronisation between the replays.
"""
import numpy as np
import pytest

import synth_inputs as SI
from parity_utils import device, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lay():
    import torch  # noqa: F401
    device()
    from hybrid_softmax_gated_amd import layer
    return layer


def _frame_inputs(w):
    import torch
    passes = list(SI.iter_passes(w, frames=1))
    dev = device()
    return [dict(q=to_dev(p.q, w.dtype), k=to_dev(p.k, w.dtype), v=to_dev(p.v, w.dtype),
                 alpha=torch.from_numpy(p.alpha).to(dev), beta=torch.from_numpy(p.beta).to(dev),
                 update=p.update) for p in passes]


@pytest.mark.parametrize("access", ["frame", "token"])
def test_captured_frame_matches_eager_on_every_replay(lay, access):
    import torch
    w = SI.companion(SI.scaled(SI.WORKLOADS["frame_step_480p"], L=400))
    W = to_dev(SI.make_weights(w), w.dtype)
    S0 = torch.from_numpy(SI.make_state0(w)).to(device())
    ins = _frame_inputs(w)
    A = lay.ARL2Layer(w.B, w.H, w.d, w.L, 0)
    B = lay.ARL2Layer(w.B, w.H, w.d, w.L, 0)
    A.reset(S0)
    B.reset(S0)
    shape = (w.B, w.L, w.H, w.d)
    outA = [torch.empty(shape, dtype=torch.bfloat16, device=device()) for _ in ins]
    outB = [torch.empty(shape, dtype=torch.bfloat16, device=device()) for _ in ins]

    def run(layer, outs, stream=None):
        for p, o in zip(ins, outs):
            if access == "token":
                layer.forward_token_level(p["q"], p["k"], p["v"], W, p["alpha"], p["beta"], o,
                                          p["update"], stream)
            else:
                layer.forward(p["q"], p["k"], p["v"], W, p["alpha"], p["beta"], o, p["update"],
                              stream)

    if access == "token":   # the token-level workspace is allocated before capture
        A.forward_token_level(ins[0]["q"], ins[0]["k"], ins[0]["v"], W, ins[0]["alpha"],
                              ins[0]["beta"], outA[0], False)
        torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run(A, outA, torch.cuda.current_stream())
    torch.cuda.synchronize()
    assert torch.equal(A.S, S0), "capturing must not run the kernels"
    for rep in range(3):
        g.replay()
        run(B, outB)
        scratch = torch.randn(1 << 20, device=device()).sum()   # eager work in between
        torch.cuda.synchronize()
        assert torch.isfinite(scratch)
        for oa, ob in zip(outA, outB):
            assert torch.equal(oa, ob), f"replay {rep}: outputs differ"
        assert torch.equal(A.S, B.S), f"replay {rep}: states differ"
    assert not torch.equal(A.S, S0)
