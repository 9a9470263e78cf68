"""A small attention-only stack mixing the hybrid layer with softmax
key/value-cache layers, against the oracle's layer-by-layer composition.

Six layers, three of them the hybrid layer ("Technical Summary: Attend
Locally, Remember Linearly (ARL2)", section 4: a share of the attention
layers replaced; section 1: the others keep a cache of every earlier frame),
2 heads of 128, 200 tokens per frame, 3 frames of 1 query-only + 1 clean
pass. Every layer gets its own seeded synthetic activations (the stack holds
no projections between layers). Per pass, every layer's output is compared
with the oracle: the hybrid layers with frame_forward on the oracle's own
state, the softmax layers with kv_cache_attention over the oracle's own
cache (the clean keys/values of the earlier frames, then the pass's own).
After every clean pass every hybrid layer's state is compared as well.
"""
import numpy as np
import pytest

import oracle as O
import synth_inputs as SI
from parity_utils import TOL_OUT, TOL_S, device, out_err_per_head, state_err, to_dev, to_host

pytestmark = pytest.mark.gpu


def test_mixed_stack_six_layers_half_replaced():
    import torch
    from hybrid_softmax_gated_amd.stack import AttentionStack

    dev = device()
    layers, n_hybrid = 6, 3
    base = SI.Workload("stack6", 1, 2, 128, 200, 3, 1, SI.BF16, 0.0)
    ws = [SI.scaled(base, seed=100 + li, name=f"stack6_layer{li}") for li in range(layers)]
    passes = [list(SI.iter_passes(w)) for w in ws]
    W = [SI.make_weights(w) for w in ws]
    Wd = [to_dev(x, SI.BF16) for x in W]
    B, H, d, L = base.B, base.H, base.d, base.L
    stack = AttentionStack(B, H, d, L, layers, n_hybrid, device=dev)
    assert [stack.kind(li) for li in range(layers)] == ["hybrid"] * 3 + ["softmax"] * 3
    S_ref = [np.zeros((B, H, d, d)) for _ in range(n_hybrid)]
    cache_ref = [{"k": [], "v": []} for _ in range(layers - n_hybrid)]
    out = torch.empty((B, L, H, d), dtype=torch.bfloat16, device=dev)
    worst_out, worst_s, checked = 0.0, 0.0, 0
    npass = base.passes_per_frame
    for f in range(base.frames):
        for ps in range(npass):
            for li in range(layers):
                p = passes[li][f * npass + ps]
                assert p.frame == f and p.index == ps
                q, k, v = (to_dev(x, SI.BF16) for x in (p.q, p.k, p.v))
                alpha = torch.from_numpy(p.alpha).to(dev)
                beta = torch.from_numpy(p.beta).to(dev)
                stack.forward(li, f, q, k, v, Wd[li], alpha, beta, out, p.update)
                torch.cuda.synchronize()
                got = to_host(out)
                if li < n_hybrid:
                    ref = O.frame_forward(p.q, p.k, p.v, W[li], S_ref[li], p.alpha, p.beta,
                                          int(p.update))
                    if p.update:
                        worst_s = max(worst_s, state_err(to_host(stack.hybrid[li].S),
                                                         S_ref[li]))
                else:
                    c = cache_ref[li - n_hybrid]
                    kc = np.concatenate(c["k"] + [p.k], axis=1)
                    vc = np.concatenate(c["v"] + [p.v], axis=1)
                    assert kc.shape[1] == (f + 1) * L
                    ref = O.kv_cache_attention(p.q, kc, vc)
                    if p.update:  # the clean pass's keys/values stay for later frames
                        c["k"].append(p.k)
                        c["v"].append(p.v)
                worst_out = max(worst_out, out_err_per_head(got, ref))
                checked += 1
    print(f"stack of {layers} layers: {checked} layer passes, max out err {worst_out:.2e}, "
          f"max S err {worst_s:.2e}")
    assert checked == layers * base.frames * npass
    assert worst_out < TOL_OUT[SI.BF16]
    assert worst_s < TOL_S
    # the hybrid layers' memory did not grow; each softmax cache holds 3 frames
    assert all(c.frames == base.frames for c in stack.caches)
