"""arl2_frame_forward_noalloc against arl2_frame_forward.

The no-allocation pass runs the same kernels with its workspace in the
library's per-device scratch array instead of the caller's workspace, so on
the same inputs its output and state must equal those of the ordinary pass
bitwise. Two calls in a row: first the 480p frame step (12 heads, 1560
tokens; a query-only and a clean pass), then a smaller frame (2 heads, 200
tokens) on a second pair of states, which also checks that what the first
call left in the scratch does not leak into the second. The states of the
no-allocation pass are bound without a workspace.
"""
import pytest

import synth_inputs as SI
from parity_utils import device, to_dev

pytestmark = pytest.mark.gpu


def _pair(Bd, torch, w):
    """(ordinary layer, no-workspace state, its S) for workload w, both
    starting from the workload's S0."""
    from hybrid_softmax_gated_amd.layer import ARL2Layer

    dev = device()
    ref = ARL2Layer(w.B, w.H, w.d, w.L, Bd.ARL2_BF16)
    S = torch.empty((w.B, w.H, w.d, w.d), dtype=torch.float32, device=dev)
    st = Bd.arl2_state()
    Bd.arl2_state_init(st, w.B, w.H, w.d, w.L, Bd.ARL2_BF16, S, None, 0, None)
    S0 = torch.from_numpy(SI.make_state0(w)).to(dev)
    ref.reset(S0)
    Bd.arl2_state_reset(st, S0, None)
    return ref, st, S


@pytest.mark.parametrize("name,w", [
    ("frame_step_480p", SI.WORKLOADS["frame_step_480p"]),
    ("small_after_large", SI.Workload("small", 1, 2, 128, 200, 1, 1, SI.BF16, 0.02, seed=5)),
])
def test_noalloc_pass_equals_the_ordinary_pass(name, w):
    import torch
    from hybrid_softmax_gated_amd import binding as Bd

    assert Bd.arl2_workspace_bytes(w.B, w.H, w.d, w.L, Bd.ARL2_BF16) <= \
        Bd.ARL2_NOALLOC_SCRATCH_BYTES
    dev = device()
    ref, st, S = _pair(Bd, torch, w)
    Wd = to_dev(SI.make_weights(w), SI.BF16)
    out_ref = torch.empty((w.B, w.L, w.H, w.d), dtype=torch.bfloat16, device=dev)
    out = torch.full_like(out_ref, float("nan"))
    for p in SI.iter_passes(w):
        q, k, v = (to_dev(x, SI.BF16) for x in (p.q, p.k, p.v))
        alpha = torch.from_numpy(p.alpha).to(dev)
        beta = torch.from_numpy(p.beta).to(dev)
        ref.forward(q, k, v, Wd, alpha, beta, out_ref, p.update)
        Bd.arl2_frame_forward_noalloc(q, k, v, Wd, st, alpha, beta, out, int(p.update), None)
        torch.cuda.synchronize()
        assert torch.equal(out, out_ref), f"{name}: output of pass {p.index} differs"
        assert torch.equal(S, ref.S), f"{name}: state after pass {p.index} differs"
    assert bool(torch.isfinite(S).all())
    # a state without a workspace is refused by the ordinary pass
    with pytest.raises(Bd.ARL2Error, match="noalloc"):
        Bd.arl2_frame_forward(q, k, v, Wd, st, alpha, beta, out, 0, None)
