"""The streaming workloads at full size on the GPU against the float64 oracle.

Inputs are drawn on the GPU (synth_inputs.iter_passes_device) and the exact
bytes are copied back for the oracle. The oracle carries its own state from
frame to frame and is never re-synced to the GPU's.

Per clean pass the whole state is compared (max-norm relative error per
(stream, head) <= 1e-3). Outputs are compared on sampled rows (first and
last rows, tile edges, random rows) of every (stream, head), computed by the
oracle one row at a time (<= 2e-2 for bf16 io).

The literal update is expansive at the 480p shape (the frame transition has
spectral radius about 10), so the 231-frame literal run is compared on the
frames before the oracle's state leaves the fp32 range, and the GPU state
must turn non-finite within one frame of that point. The companion runs
(beta / L) keep the state bounded and are compared on every frame.
"""
import time

import numpy as np
import pytest

import oracle as O
import synth_inputs as SI
from parity_utils import (TOL_OUT, TOL_S, device, oracle_clock, oracle_state_update,
                          out_err_per_head, sample_rows, state_err, to_dev, to_host)

pytestmark = pytest.mark.gpu

FP32_MAX = float(np.finfo(np.float32).max)


@pytest.fixture(scope="module")
def torch():
    import torch as t
    device()
    return t


@pytest.fixture(scope="module")
def lay(torch):
    from hybrid_softmax_gated_amd import layer
    return layer


def _oracle_rows(q_rows, k, v, W, S):
    """Oracle output of the sampled query rows q_rows [B][R][H][d] of every
    (stream, head) over the whole frame k, v [B][L][H][d]."""
    B, R, H, d = q_rows.shape
    out = np.empty((B, R, H, d))
    for b in range(B):
        for h in range(H):
            out[b, :, h] = O.output_rows(q_rows[b, :, h], k[b, :, h], v[b, :, h], W[0, h],
                                         S[b, h], np.arange(R))
    return out


def _stream(lay, torch, w, frames=None, rows_n=12, out_every=1, until_overflow=False,
            full_at=(), full_errs=None):
    """Runs a workload; returns per-clean-pass records and the output errors.

    out_every: compare sampled outputs on every pass (1) or on the first
    query-only pass and the clean pass of every frame (0).
    full_at: (frame, pass index) pairs, 0-based, whose whole output (every
    row of every (stream, head)) is compared with the oracle; the worst
    per-(stream, head) error of each is appended to ``full_errs``."""
    layer = lay.ARL2Layer(w.B, w.H, w.d, w.L, 0)
    W = SI.make_weights(w)
    Wd = to_dev(W, w.dtype)
    S_ref = SI.make_state0(w).astype(np.float64)
    if np.any(S_ref):
        layer.reset(torch.from_numpy(S_ref.astype(np.float32)).to(device()))
    out = torch.empty((w.B, w.L, w.H, w.d), dtype=SI.torch_dtype(w.dtype), device=device())
    rows = sample_rows(w.L, rows_n, w.seed + 7)
    rows_t = torch.from_numpy(rows).to(device())
    recs, out_errs, mem = [], [], []
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    frame_ms, t_frame = [], 0.0
    for p in SI.iter_passes_device(w, device(), frames):
        ref_finite = bool(np.max(np.abs(S_ref)) < FP32_MAX)
        ev[0].record()
        layer.forward(p.q, p.k, p.v, Wd, p.alpha, p.beta, out, p.update, gate=w.gate)
        ev[1].record()
        torch.cuda.synchronize()
        t_frame += ev[0].elapsed_time(ev[1])
        check_out = ref_finite and (out_every == 1 or p.index == 0 or p.update)
        full = ref_finite and (p.frame, p.index) in full_at
        if check_out or p.update or full:
            k = p.k.float().cpu().numpy()
            v = p.v.float().cpu().numpy()
        if full:
            q = p.q.float().cpu().numpy()
            got_full = to_host(out)
            ref_full = np.empty_like(got_full)
            with oracle_clock(w.name + "_full_outputs"):
                for b in range(w.B):
                    for h in range(w.H):
                        ref_full[b, :, h] = O.output_rows(q[b, :, h], k[b, :, h], v[b, :, h],
                                                          W[0, h], S_ref[b, h], np.arange(w.L))
            full_errs.append(((p.frame, p.index), out_err_per_head(got_full, ref_full)))
            del q, got_full, ref_full
        if check_out:
            q_rows = p.q.index_select(1, rows_t).float().cpu().numpy()
            got = out.index_select(1, rows_t).float().cpu().numpy().astype(np.float64)
            with oracle_clock(w.name):
                ref_rows = _oracle_rows(q_rows, k, v, W, S_ref)
            out_errs.append((p.frame, out_err_per_head(got, ref_rows)))
        if p.update:
            # the same tensors are alive at every clean pass: the library
            # itself allocates nothing. The sum of the live requests is
            # compared, not the caching allocator's block sizes, which it may
            # round up by a cached block's unsplit remainder.
            mem.append(torch.cuda.memory_stats()["requested_bytes.all.current"])
            frame_ms.append(t_frame)
            t_frame = 0.0
            alpha_h, beta_h = p.alpha.cpu().numpy(), p.beta.cpu().numpy()
            with oracle_clock(w.name):
                oracle_state_update(S_ref, k, v, W, alpha_h, beta_h)
            S_gpu = to_host(layer.S)
            rec = {"frame": p.frame, "ref_finite": bool(np.max(np.abs(S_ref)) < FP32_MAX),
                   "gpu_finite": bool(np.all(np.isfinite(S_gpu))),
                   "norm": float(np.max(np.abs(S_ref)))}
            if rec["ref_finite"] and rec["gpu_finite"]:
                rec["err"] = state_err(S_gpu, S_ref)
            recs.append(rec)
            if until_overflow and not rec["ref_finite"] and not rec["gpu_finite"]:
                break
    assert len(set(mem)) == 1, f"device memory changed across frames: {sorted(set(mem))}"
    return recs, out_errs, frame_ms


def _check(recs, out_errs, name, before_frame=None):
    if before_frame is not None:
        recs = [r for r in recs if r["frame"] < before_frame]
        out_errs = [e for e in out_errs if e[0] < before_frame]
    out_errs = [e for _, e in out_errs]
    errs = [r["err"] for r in recs if "err" in r]
    print(f"{name}: {len(recs)} clean passes, max S err {max(errs):.2e}, "
          f"{len(out_errs)} passes with sampled outputs, max out err {max(out_errs):.2e}, "
          f"final max|S| {recs[-1]['norm']:.3e}")
    assert max(errs) < TOL_S
    assert max(out_errs) < TOL_OUT[SI.BF16]


@pytest.mark.parametrize("companion", [False, True])
def test_stream21_480p(lay, torch, companion):
    """21 latent frames, 4 query-only passes + 1 clean pass each, fresh
    q, k, v every pass, state carried across frames from S0 = 0."""
    w = SI.WORKLOADS["stream21_480p"]
    w = SI.companion(w) if companion else w
    recs, out_errs, _ = _stream(lay, torch, w)
    assert len(recs) == 21 and all(r["gpu_finite"] and r["ref_finite"] for r in recs)
    _check(recs, out_errs, w.name)


def test_stream21_480p_elementwise_gate(lay, torch):
    """The 21-frame stream with the ablation's elementwise forget gate (one
    value per d_k row, alpha = sigmoid(N(2, 0.5)) per element)."""
    w = SI.scaled(SI.WORKLOADS["stream21_480p"], gate="elementwise", name="stream21_480p_elementwise")
    recs, out_errs, _ = _stream(lay, torch, w)
    assert len(recs) == 21 and all(r["gpu_finite"] and r["ref_finite"] for r in recs)
    _check(recs, out_errs, w.name)


def test_long231_480p_beta_over_L(lay, torch):
    """231 frames (one query-only + one clean pass each) with the bounded
    companion gates: the state is compared on every frame, device memory
    stays constant, and the per-frame GPU time does not grow with the frame
    index."""
    w = SI.companion(SI.WORKLOADS["long231_480p"])
    recs, out_errs, frame_ms = _stream(lay, torch, w, rows_n=8)
    assert len(recs) == 231
    _check(recs, out_errs, w.name)
    first, last = np.median(frame_ms[5:35]), np.median(frame_ms[-30:])
    print(f"GPU ms per frame: frames 6-35 median {first:.4f}, last 30 median {last:.4f}")
    assert last < 1.5 * first


def test_long231_480p_literal(lay, torch):
    """The literal gates: compared frame by frame until the oracle's state
    leaves the fp32 range; the GPU's state must turn non-finite within one
    frame of that point (fp32 cannot hold it, the float64 oracle can)."""
    w = SI.WORKLOADS["long231_480p"]
    recs, out_errs, _ = _stream(lay, torch, w, rows_n=8, until_overflow=True)
    first_ref = next((r["frame"] for r in recs if not r["ref_finite"]), None)
    first_gpu = next((r["frame"] for r in recs if not r["gpu_finite"]), None)
    print(f"oracle state leaves fp32 range at frame {first_ref}, GPU state non-finite at "
          f"frame {first_gpu}")
    assert first_ref is not None and first_gpu is not None
    assert abs(first_gpu - first_ref) <= 1
    _check(recs, out_errs, w.name, before_frame=min(first_ref, first_gpu))


def test_maximum_frame_length(lay, torch):
    """The longest frame the library accepts (ARL2_MAX_L = 2^20 tokens, one
    head): one query-only and one clean pass. The attention then runs every
    query block over all 16,384 key tiles in one key range, and the state
    update sums 8,192 chunk contributions; the whole state and sampled output
    rows are compared with the oracle."""
    w = SI.Workload("max_frame_length", 1, 1, 128, 1 << 20, 1, 1, SI.BF16, 0.02, seed=2020)
    t0 = time.time()
    recs, out_errs, _ = _stream(lay, torch, w, rows_n=8)
    print(f"maximum frame length took {time.time() - t0:.1f} s")
    assert len(recs) == 1 and recs[0]["gpu_finite"] and recs[0]["ref_finite"]
    _check(recs, out_errs, w.name)


@pytest.mark.parametrize("Bn,H", [(1, 65535), (65535, 1)])
def test_maximum_heads_and_streams(lay, torch, Bn, H):
    """The largest head count and stream count accepted (65,535), each with a
    64-token frame: one query-only and one clean pass. Inputs are drawn on
    the GPU; the first, last and middle (stream, head) pairs are checked
    against the oracle (outputs on every pass, the state after the clean
    pass), so every index of the large dimension's extremes is exercised."""
    L, d = 64, 128
    dev = device()
    g = torch.Generator(device=dev)
    g.manual_seed(Bn * 7 + H)
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
        layer.forward(q, k, v, W, alpha, beta, out, update)
        torch.cuda.synchronize()
        for b, h in pairs:
            def one(t):
                return t[b:b + 1, :, h:h + 1].float().cpu().numpy()
            Sh = S_ref[(b, h)][None, None].copy()
            ref = O.frame_forward(one(q), one(k), one(v), W[:, h:h + 1].float().cpu().numpy(), Sh,
                                  alpha[b:b + 1, h:h + 1].cpu().numpy(),
                                  beta[b:b + 1, :, h:h + 1].cpu().numpy(), update)
            got = one(out).astype(np.float64)
            err = np.max(np.abs(got - ref)) / np.max(np.abs(ref))
            assert err < TOL_OUT[SI.BF16], (b, h, update, err)
            if update:
                S_ref[(b, h)] = Sh[0, 0]
    for b, h in pairs:
        ref = S_ref[(b, h)]
        err = np.max(np.abs(layer.S[b, h].double().cpu().numpy() - ref)) / np.max(np.abs(ref))
        assert err < TOL_S, (b, h, err)


def test_batched720p(lay, torch):
    """Four independent streams (seeds 0..3) at the 720p latent shape
    (L = 3600), 21 frames of 4 query-only + 1 clean pass; sampled outputs
    on every pass, and every output row of every (stream, head) on the first
    query-only pass of frame 1 and the clean passes of frames 1 and 21. This
    shape's plan differs from 480p's: one key range of 57 tiles per query
    block, 29 query blocks per head and 128-token update chunks."""
    w = SI.WORKLOADS["batched720p"]
    t0 = time.time()
    full = []
    recs, out_errs, _ = _stream(lay, torch, w, rows_n=8, full_at={(0, 0), (0, 4), (20, 4)},
                                full_errs=full)
    print(f"batched720p took {time.time() - t0:.1f} s; full outputs (frame, pass): "
          + ", ".join(f"{fp}: {e:.2e}" for fp, e in full))
    assert len(recs) == 21
    assert sorted(fp for fp, _ in full) == [(0, 0), (0, 4), (20, 4)]
    assert max(e for _, e in full) < TOL_OUT[SI.BF16]
    _check(recs, out_errs, w.name)


def test_kv_cache_attention_at_231_frames(lay, torch):
    """The comparator at the long horizon's end: one frame's queries (12
    heads, L = 1560) over a cache of 231 frames (360,360 keys), on sampled
    rows."""
    B, H, d, Lq = 1, 12, 128, 1560
    Lk = 231 * Lq
    g = torch.Generator(device=device())
    g.manual_seed(231)
    q = torch.randn((B, Lq, H, d), generator=g, device=device()).to(torch.bfloat16)
    kc = torch.randn((B, Lk, H, d), generator=g, device=device()).to(torch.bfloat16)
    vc = torch.randn((B, Lk, H, d), generator=g, device=device()).to(torch.bfloat16)
    out = torch.empty_like(q)
    lay.softmax_attention(q, kc, vc, out, 0)
    torch.cuda.synchronize()
    rows = sample_rows(Lq, 6, 5)
    got = to_host(out)[0, rows]
    qh = q.float().cpu().numpy()[0, rows]
    for h in range(H):
        ref = O.intra_attention(qh[:, h].astype(np.float64),
                                kc[0, :, h].float().cpu().numpy().astype(np.float64),
                                vc[0, :, h].float().cpu().numpy().astype(np.float64))
        err = float(np.max(np.abs(got[:, h] - ref)) / np.max(np.abs(ref)))
        assert err < TOL_OUT[SI.BF16], (h, err)
