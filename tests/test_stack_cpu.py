"""Bookkeeping of the attention-only stack's key/value caches, on CPU
tensors (no kernels): slot order, overwrites within a frame, capacity
doubling that keeps earlier frames, and contiguous per-stream views."""
import pytest
import torch

from hybrid_softmax_gated_amd.stack import AttentionStack, KVCache


def _kv(Bn, L, H, d, tag):
    k = torch.full((Bn, L, H, d), float(tag))
    k += torch.arange(Bn).view(Bn, 1, 1, 1) * 1000
    return k, -k


def test_cache_holds_the_last_pass_of_each_frame_and_grows_by_doubling():
    Bn, L, H, d = 2, 5, 3, 4
    c = KVCache(Bn, L, H, d, torch.float32, "cpu")
    caps = []
    for f in range(6):
        for ps in range(3):  # three passes per frame; the last one stays
            k, v = _kv(Bn, L, H, d, 10 * f + ps)
            c.write(f, k, v)
            assert c.frames == f + 1
        caps.append(c.capacity)
        for b in range(Bn):
            kb, vb = c.keys(b), c.values(b)
            assert kb.shape == (1, (f + 1) * L, H, d) and kb.is_contiguous() and vb.is_contiguous()
            for g in range(f + 1):
                want = 10 * g + 2 + 1000 * b
                assert torch.all(kb[0, g * L:(g + 1) * L] == want)
                assert torch.all(vb[0, g * L:(g + 1) * L] == -want)
    assert caps == [1, 2, 4, 4, 8, 8]


def test_cache_rejects_out_of_order_frames():
    c = KVCache(1, 4, 1, 2, torch.float32, "cpu")
    k, v = _kv(1, 4, 1, 2, 0)
    c.write(0, k, v)
    with pytest.raises(ValueError):
        c.write(2, k, v)
    c.write(1, k, v)
    with pytest.raises(ValueError):
        c.write(0, k, v)


def test_stack_layer_kinds():
    with pytest.raises(ValueError):
        AttentionStack(1, 1, 128, 64, 4, 5, device="cpu")
