"""HIP path vs the float64 oracle through the C ABI, on identical seeded bytes.

Bar: outputs within 2e-2 (bf16 io) / 1e-4 (fp32 io) max-norm relative error
per (stream, head) and pass; state within 1e-3 per (stream, head); integer
work (tiling, ragged tails) is covered by ragged sizes that must meet the
same bar everywhere, including the last partial tile.
"""
import os

import numpy as np
import pytest

import oracle as O
import synth_inputs as SI
from parity_utils import (TOL_OUT, TOL_S, device, oracle_clock, oracle_rows,
                          oracle_state_update, out_err_per_head, rel_max_err, sample_rows,
                          state_err, to_dev, to_host)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch():
    import torch as t
    device()
    return t


@pytest.fixture(scope="module")
def lay(torch):
    from hybrid_softmax_gated_amd import layer
    return layer


def _run_stream(lay, torch, w, frames=None, S0=None, check_every_pass=True):
    """Run a whole workload on the GPU and the oracle (full outputs)."""
    dtype = 0 if w.dtype == SI.BF16 else 1
    L = lay.ARL2Layer(w.B, w.H, w.d, w.L, dtype)
    W = SI.make_weights(w)
    Wd = to_dev(W, w.dtype)
    S_ref = (SI.make_state0(w) if S0 is None else S0).astype(np.float64)
    if np.any(S_ref):
        L.reset(torch.from_numpy(S_ref.astype(np.float32)).to(device()))
    errs_out, errs_s = [], []
    out = torch.empty((w.B, w.L, w.H, w.d), dtype=SI.torch_dtype(w.dtype), device=device())
    for p in SI.iter_passes(w, frames):
        q, k, v = (to_dev(x, w.dtype) for x in (p.q, p.k, p.v))
        al = torch.from_numpy(p.alpha).to(device())
        be = torch.from_numpy(p.beta).to(device())
        L.forward(q, k, v, Wd, al, be, out, p.update, gate=w.gate)
        with oracle_clock(w.name):
            ref = O.frame_forward(p.q, p.k, p.v, W, S_ref, p.alpha, p.beta, int(p.update))
        torch.cuda.synchronize()
        if check_every_pass or p.update:
            errs_out.append(out_err_per_head(to_host(out), ref))
        if p.update:
            errs_s.append(state_err(to_host(L.S), S_ref))
    return errs_out, errs_s, L, S_ref


def test_native_library_is_loaded(torch):
    from hybrid_softmax_gated_amd import binding
    maps = open("/proc/self/maps").read()
    assert binding.LIB_PATH in maps
    hips = {ln.split()[-1] for ln in maps.splitlines() if "libamdhip64" in ln}
    assert len(hips) == 1, f"more than one HIP runtime in the process: {hips}"


def test_tiny_f32_stream(lay, torch):
    w = SI.WORKLOADS["tiny_f32"]
    eo, es, _, _ = _run_stream(lay, torch, w)
    print("tiny_f32 out errs", eo, "S errs", es)
    assert max(eo) < TOL_OUT[SI.F32]
    assert max(es) < TOL_S


@pytest.mark.parametrize("L", [1, 37, 64, 100, 129, 255, 1560])
def test_intra_branch_alone_bf16(lay, torch, L):
    """S = 0: the output is the intra-frame branch alone, so errors of the
    softmax attention are not hidden behind a large O_inter."""
    H = 12 if L == 1560 else 2
    w = SI.Workload("intra", 1, H, 128, L, 1, 0, SI.BF16, 0.0, seed=L)
    eo, _, _, _ = _run_stream(lay, torch, SI.scaled(w), check_every_pass=True)
    print(f"L={L} intra-only err {eo}")
    assert max(eo) < TOL_OUT[SI.BF16]


def test_frame_step_480p(lay, torch):
    """One Wan2.1-1.3B frame step: 12 heads x 128, L = 1560, warm state,
    one query-only pass and one clean pass (full outputs and state)."""
    w = SI.WORKLOADS["frame_step_480p"]
    eo, es, _, _ = _run_stream(lay, torch, w)
    print("frame_step_480p out errs", eo, "S errs", es)
    assert max(eo) < TOL_OUT[SI.BF16]
    assert max(es) < TOL_S


@pytest.mark.parametrize("B,H,L", [(2, 3, 200), (3, 1, 1000), (1, 2, 130)])
def test_batched_ragged_bf16(lay, torch, B, H, L):
    w = SI.Workload("ragged", B, H, 128, L, 3, 1, SI.BF16, 0.02, seed=B * 100 + L)
    eo, es, _, _ = _run_stream(lay, torch, w)
    print(f"B={B} H={H} L={L} out {max(eo):.2e} S {max(es):.2e}")
    assert max(eo) < TOL_OUT[SI.BF16]
    assert max(es) < TOL_S


@pytest.mark.parametrize("dtype,d,L", [(SI.BF16, 16, 50), (SI.F32, 128, 70), (SI.F32, 16, 1)])
def test_generic_paths(lay, torch, dtype, d, L):
    w = SI.Workload("generic", 2, 2, d, L, 3, 1, dtype, 0.02, seed=d + L)
    eo, es, _, _ = _run_stream(lay, torch, w)
    print(f"{dtype} d={d} L={L} out {max(eo):.2e} S {max(es):.2e}")
    assert max(eo) < TOL_OUT[dtype]
    assert max(es) < TOL_S


@pytest.mark.parametrize("dtype,d,B,H,L", [(SI.BF16, 128, 2, 3, 200), (SI.F32, 16, 2, 2, 50),
                                           (SI.BF16, 128, 1, 12, 1560)])
def test_elementwise_gate(lay, torch, dtype, d, B, H, L):
    """The ablation's elementwise forget gate (one value per d_k row), on the
    MFMA path (bf16, d = 128) and the generic path (f32, d = 16)."""
    w = SI.Workload("gate", B, H, d, L, 3, 1, dtype, 0.02, seed=d + L, gate="elementwise")
    eo, es, _, _ = _run_stream(lay, torch, w)
    print(f"elementwise gate {dtype} d={d} L={L}: out {max(eo):.2e} S {max(es):.2e}")
    assert max(eo) < TOL_OUT[dtype]
    assert max(es) < TOL_S


def test_elementwise_gate_with_equal_entries_matches_headwise_bitwise(lay, torch):
    B, H, d, L = 2, 3, 128, 300
    p, W, (q, k, v, Wd), al, be = _one_pass_inputs(torch, B, H, d, L, SI.BF16, 21)
    res = []
    for gate in ("headwise", "elementwise"):
        layer = lay.ARL2Layer(B, H, d, L, 0)
        layer.reset(torch.full((B, H, d, d), 0.01, device=device()))
        a = al if gate == "headwise" else al[:, :, None].expand(B, H, d).contiguous()
        out = torch.empty((B, L, H, d), dtype=torch.bfloat16, device=device())
        layer.forward(q, k, v, Wd, a, be, out, True, gate=gate)
        torch.cuda.synchronize()
        res.append(layer.S.clone())
    assert torch.equal(res[0].view(torch.int32), res[1].view(torch.int32))


def _one_pass_inputs(torch, B, H, d, L, dtype, seed):
    p = SI.random_pass(B, H, d, L, dtype, seed)
    W = SI.make_weights(SI.Workload("w", B, H, d, L, 1, 0, dtype, 0.0, seed=seed))
    dev = [to_dev(x, dtype) for x in (p.q, p.k, p.v, W)]
    al = torch.from_numpy(p.alpha).to(device())
    be = torch.from_numpy(p.beta).to(device())
    return p, W, dev, al, be


def test_noisy_pass_leaves_state_bitwise(lay, torch):
    B, H, d, L = 1, 4, 128, 300
    p, W, (q, k, v, Wd), al, be = _one_pass_inputs(torch, B, H, d, L, SI.BF16, 3)
    layer = lay.ARL2Layer(B, H, d, L, 0)
    S0 = torch.randn((B, H, d, d), device=device()) * 0.02
    layer.reset(S0)
    out = torch.empty((B, L, H, d), dtype=torch.bfloat16, device=device())
    before = layer.S.clone()
    layer.forward(q, k, v, Wd, None, None, out, False)
    torch.cuda.synchronize()
    assert torch.equal(layer.S.view(torch.int32), before.view(torch.int32))


def test_alpha_one_beta_zero_leaves_state_bitwise(lay, torch):
    B, H, d, L = 2, 2, 128, 257
    p, W, (q, k, v, Wd), al, be = _one_pass_inputs(torch, B, H, d, L, SI.BF16, 4)
    layer = lay.ARL2Layer(B, H, d, L, 0)
    layer.reset(torch.randn((B, H, d, d), device=device()))
    out = torch.empty((B, L, H, d), dtype=torch.bfloat16, device=device())
    before = layer.S.clone()
    layer.forward(q, k, v, Wd, torch.ones_like(al), torch.zeros_like(be), out, True)
    torch.cuda.synchronize()
    assert torch.equal(layer.S.view(torch.int32), before.view(torch.int32))


def test_zero_state_output_is_intra_branch_and_clean_pass_reads_old_state(lay, torch):
    B, H, d, L = 1, 3, 128, 400
    p, W, (q, k, v, Wd), al, be = _one_pass_inputs(torch, B, H, d, L, SI.BF16, 5)
    layer = lay.ARL2Layer(B, H, d, L, 0)
    out_n = torch.empty((B, L, H, d), dtype=torch.bfloat16, device=device())
    out_c = torch.empty_like(out_n)
    layer.forward(q, k, v, Wd, None, None, out_n, False)
    layer.forward(q, k, v, Wd, al, be, out_c, True)
    torch.cuda.synchronize()
    # same pre-update state for both passes -> identical bits
    assert torch.equal(out_n.view(torch.int16), out_c.view(torch.int16))
    ref = O.kv_cache_attention(p.q, p.k, p.v)
    assert out_err_per_head(to_host(out_n), ref) < TOL_OUT[SI.BF16]
    assert torch.any(layer.S != 0)


def test_runs_are_bitwise_reproducible(lay, torch):
    B, H, d, L = 1, 12, 128, 1560
    p, W, (q, k, v, Wd), al, be = _one_pass_inputs(torch, B, H, d, L, SI.BF16, 6)
    res = []
    for _ in range(2):
        layer = lay.ARL2Layer(B, H, d, L, 0)
        layer.reset(torch.ones((B, H, d, d), device=device()) * 0.01)
        out = torch.empty((B, L, H, d), dtype=torch.bfloat16, device=device())
        layer.forward(q, k, v, Wd, al, be, out, True)
        layer.forward(q, k, v, Wd, al, be, out, True)
        torch.cuda.synchronize()
        res.append((out.clone(), layer.S.clone()))
    assert torch.equal(res[0][0].view(torch.int16), res[1][0].view(torch.int16))
    assert torch.equal(res[0][1].view(torch.int32), res[1][1].view(torch.int32))


def test_token_permutation(lay, torch):
    """Frame-level access: permuting the tokens of a frame permutes the
    outputs and leaves the updated state unchanged (within rounding)."""
    B, H, d, L = 1, 2, 128, 333
    p, W, (q, k, v, Wd), al, be = _one_pass_inputs(torch, B, H, d, L, SI.BF16, 8)
    perm = torch.from_numpy(np.random.default_rng(9).permutation(L)).to(device())
    res = []
    for idx in (None, perm):
        layer = lay.ARL2Layer(B, H, d, L, 0)
        layer.reset(torch.full((B, H, d, d), 0.01, device=device()))
        qq, kk, vv, bb_ = (x if idx is None else x[:, idx].contiguous() for x in (q, k, v, be))
        out = torch.empty((B, L, H, d), dtype=torch.bfloat16, device=device())
        layer.forward(qq, kk, vv, Wd, al, bb_, out, True)
        torch.cuda.synchronize()
        res.append((to_host(out), to_host(layer.S)))
    assert rel_max_err(res[1][0], res[0][0][:, perm.cpu().numpy()]) < 1e-2
    assert state_err(res[1][1], res[0][1]) < 1e-4


def test_state_reset_restores_a_saved_stream(lay, torch):
    """Checkpoint/resume: copying S out after frame k and restoring it with
    arl2_state_reset gives the same bits as an uninterrupted stream."""
    w = SI.Workload("resume", 1, 2, 128, 150, 4, 1, SI.BF16, 0.0, seed=12)
    W = SI.make_weights(w)
    Wd = to_dev(W, w.dtype)
    passes = list(SI.iter_passes(w))
    dev = [(to_dev(p.q, w.dtype), to_dev(p.k, w.dtype), to_dev(p.v, w.dtype),
            torch.from_numpy(p.alpha).to(device()), torch.from_numpy(p.beta).to(device()), p.update)
           for p in passes]
    out = torch.empty((1, 150, 2, 128), dtype=torch.bfloat16, device=device())
    a = lay.ARL2Layer(1, 2, 128, 150, 0)
    for i, (q, k, v, al, be, up) in enumerate(dev):
        a.forward(q, k, v, Wd, al, be, out, up)
        if i == 3:
            saved = a.S.clone()
    b = lay.ARL2Layer(1, 2, 128, 150, 0)
    b.reset(saved)
    for (q, k, v, al, be, up) in dev[4:]:
        b.forward(q, k, v, Wd, al, be, out, up)
    torch.cuda.synchronize()
    assert torch.equal(a.S.view(torch.int32), b.S.view(torch.int32))


@pytest.mark.parametrize("Lq,Lk", [(200, 700), (64, 1), (1560, 4680)])
def test_kv_cache_attention(lay, torch, Lq, Lk):
    """The comparator: one frame's queries over a key/value cache."""
    B, H, d = 1, 12 if Lq == 1560 else 2, 128
    r = np.random.default_rng(Lq + Lk)
    q = SI.round_f32_to_bf16_values(r.standard_normal((B, Lq, H, d), dtype=np.float32))
    kc = SI.round_f32_to_bf16_values(r.standard_normal((B, Lk, H, d), dtype=np.float32))
    vc = SI.round_f32_to_bf16_values(r.standard_normal((B, Lk, H, d), dtype=np.float32))
    out = torch.empty((B, Lq, H, d), dtype=torch.bfloat16, device=device())
    lay.softmax_attention(to_dev(q, SI.BF16), to_dev(kc, SI.BF16), to_dev(vc, SI.BF16), out, 0)
    torch.cuda.synchronize()
    got = to_host(out)
    rows = sample_rows(Lq, 48, Lq) if Lq > 256 else np.arange(Lq)
    for h in range(H):
        ref = O.intra_attention(q[0, rows, h].astype(np.float64), kc[0, :, h].astype(np.float64),
                                vc[0, :, h].astype(np.float64))
        assert rel_max_err(got[0, rows, h], ref) < TOL_OUT[SI.BF16]
