#!/usr/bin/env python3
"""Throughput of one ARL2 hybrid attention layer on one MI355X.

One step = one latent frame through one layer: every pass of the frame (the
query-only denoising passes, then the clean pass that updates the state),
i.e. every step of the hot path: intra-frame softmax attention, feature maps
with L2 norms, the frame-level read of the state, the combine, and the gated
delta update. Default workload: the 21-frame stream's schedule at the
Wan2.1-1.3B 480p shape (B=1, 12 heads of 128, L=1560 tokens, 4 query-only +
1 clean pass per frame); the same line also carries the 1 + 1 schedule of
the single 480p frame step (`frame_step_1p1`).

Inputs are synthetic and seeded (q, k, v ~ N(0,1) in bf16, W = I + N(0,0.01),
alpha = sigmoid(N(2,0.5)), beta = sigmoid(N(0,1)) / L so that the state stays
finite over thousands of back-to-back frames; the work does not depend on the
values). A set of distinct frames is drawn on the GPU before timing and
cycled; everything is resident in HBM when the timed region starts.

Prints one JSON line with, besides frames/s:
  frame_latency  median, 10th and 90th percentile of 200 frames each timed
                 with its own pair of HIP events, after 10 warm-up frames;
  kernels_us     per launch kind, in sequence: HIP events taken from the
                 kernels' own start and end (arl2_profile_enable with
                 repeat 1); kernels_us_warm: the same launches repeated 10
                 times back to back between two event markers;
  roofline       the dominant kernel (intra-frame attention, the query-only
                 pass's first launch) against the bf16 dense MFMA peak, from
                 its in-sequence launch time; `traffic` is the HBM bytes per
                 launch from the committed rocprofv3 counter summary when it
                 was taken on the current kernel source, else null;
  delta_update   the gated delta update's algorithmic flops over the time its
                 chunks add to the launch they share with the attention;
  epilogues      the memory-bound second launches against the HBM peak,
                 priced by the method's own bytes (inputs read once, outputs
                 written once; the design's scratch reported beside them);
  mfma_loop_peak_tflops  the bf16 MFMA rate a pure matrix-core loop sustains
                 on this device in the same run (arl2_profile_mfma_peak);
  cpu_baseline   the float64 oracle on this host's cores, on a bounded sample
                 (frames/s, and GFLOP/s on the same flop count as the GPU
                 figure; cores = the BLAS threads it used).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "hybrid-layer frames/sec + TFLOP/s (% MFMA peak), L=1560 d=128 12 heads"
PEAK_BF16_TFLOPS = 2516.6      # MI355X dense bf16 MFMA: 256 CU x 4 SIMD x 1024 flop/clk x 2.4 GHz
PEAK_HBM_GBS = 8000.0
NUM_DISTINCT_FRAMES = 8


def flops(B, H, d, L):
    """Algorithmic MFMA-eligible flops: intra attention (QK^T and PV),
    phi_q + read, and the delta update (phi_k, phi_v, K'S, K'^T R)."""
    fa = 4.0 * B * H * L * L * d
    fb = 4.0 * B * H * L * d * d
    fc = 8.0 * B * H * L * d * d
    return fa, fb, fc


def source_digest(*names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "hybrid_softmax_gated_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel, workload, digest):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if
    it was taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("source_digest") != digest:
        return None
    return t.get("bytes_per_launch")


def launch_counters(workload):
    """Per-launch counter figures (HBM bytes, MfmaUtil) from the committed
    rocprofv3 summary of this workload, keyed by launch name, for the launches
    whose sources are unchanged since; {} if there is none."""
    path = os.path.join(ROOT, "profiles", f"frame_launches_{workload}_counters.json")
    if not os.path.exists(path):
        return {}
    with open(path) as f:
        t = json.load(f)
    first = source_digest("attn.hip", "arl2_device.h", "delta_chunk.h")
    second = source_digest("frame_tail.hip", "arl2_device.h")
    ok = {"attn_partial": t["source_digests"]["first_launch"] == first,
          "attn_delta": t["source_digests"]["first_launch"] == first,
          "combine": t["source_digests"]["second_launch"] == second,
          "combine_apply": t["source_digests"]["second_launch"] == second}
    out = {k: v for k, v in t["launches"].items() if ok.get(k)}
    if out:
        out["mfma_loop_util_pct"] = t["mfma_loop_util_pct"]
    return out


def workspace_parts(B, H, d, L):
    """Bytes of the workspace regions one pass of the bf16 d = 128 path keeps
    between its launches: the key-range partials (bf16 O/l, then fp32 max
    and sum per query), the delta chunks' fp32 d x d contributions, and the
    bf16 copy of the state. The key-range count follows the attention plan
    (two workgroups per CU, at least two 64-key tiles per range, at most 8
    ranges); the chunks hold 96 tokens when the delta chunks and the
    combine's query blocks fit 512 workgroups, else 128."""
    nqblk = -(-L // 128)
    base = B * H * nqblk
    ns = max(1, min(512 // base, -(-L // 128), 8))
    kps = -(-(-(-L // ns)) // 64) * 64
    nsplit = -(-L // kps)
    blocks = B * H * nqblk * nsplit
    chunk = 96 if B * H * (-(-L // 96) + nqblk) <= 512 else 128
    nchunk = -(-L // chunk)
    return (blocks * 128 * d * 2, blocks * 128 * 2 * 4, B * H * nchunk * d * d * 4,
            B * H * d * d * 2)


def method_bytes(B, H, d, L):
    """Bytes each launch of a pass must move by the method's definition
    (each input read once, each output written once), and the scratch the
    design moves besides (written by the first launch, read by the second).
    First launch: q, k, v (and, clean pass, W_k, W_v, S, beta for the delta
    chunks). Second launch: the inter-frame read and the output, q, W_q, S,
    out (and, clean pass, S read and written by the update, alpha)."""
    o_bytes, ml_bytes, ds, s16 = workspace_parts(B, H, d, L)
    io = B * L * H * d * 2
    state = B * H * d * d * 4
    w = H * d * d * 2
    combine = io + w + state + io
    return {"attn_partial": {"method": 3 * io, "scratch": o_bytes + ml_bytes + s16},
            "attn_delta": {"method": 3 * io + 2 * w + state + B * L * H * 4,
                           "scratch": o_bytes + ml_bytes + s16 + ds},
            "combine": {"method": combine, "scratch": o_bytes + ml_bytes + s16},
            "combine_apply": {"method": combine + 2 * state + B * H * 4,
                              "scratch": o_bytes + ml_bytes + s16 + ds}}


def cpu_baseline(frames_host, W, w, budget_s=15.0, max_frames=400, access="frame"):
    """Time the float64 oracle on host copies of the same frames. Workloads
    whose full frame would not fit the budget are timed on one (stream,
    head) of each pass and scaled by the number of (stream, head) pairs."""
    import numpy as np
    import oracle as O
    fwd = O.token_level_frame_forward if access == "token" else O.frame_forward
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover - threadpoolctl is optional
        threads = os.cpu_count() or 1
    Wf = W.astype(np.float64)
    one_head = w.B * w.L > 1560
    S = np.zeros((1, 1, w.d, w.d)) if one_head else np.zeros((w.B, w.H, w.d, w.d))
    done = 0
    t0 = time.perf_counter()
    while done < max_frames and (time.perf_counter() - t0) < budget_s:
        for p in frames_host[done % len(frames_host)]:
            if one_head:
                sl = (slice(0, 1), slice(None), slice(0, 1))
                fwd(p["q"][sl], p["k"][sl], p["v"][sl], Wf[:, 0:1], S, p["alpha"][0:1, 0:1],
                    p["beta"][0:1, :, 0:1], int(p["update"]))
            else:
                fwd(p["q"], p["k"], p["v"], Wf, S, p["alpha"], p["beta"], int(p["update"]))
        done += 1
    dt = time.perf_counter() - t0
    scale = w.B * w.H if one_head else 1
    what = (f"one (stream, head) of {done} frames, scaled by {scale}" if one_head
            else f"{done} full frames, all {w.B * w.H} (stream, head) pairs")
    fa, fb, fc = flops(w.B, w.H, w.d, w.L)
    fps = done / dt / scale
    return {"value": fps, "unit": "frames/s", "cores": int(threads), "kind": "oracle",
            "gflops": round(fps * (w.passes_per_frame * (fa + fb) + fc) / 1e9, 2),
            "host_cpu_count": os.cpu_count(),
            "sample": f"{what} ({w.noisy_passes} query-only + 1 clean pass each) of {w.name}, "
                      f"float64 NumPy/OpenBLAS, {dt:.1f} s"}


def per_frame_report(path):
    """Long horizon: per-frame GPU latency and device memory of the layer and
    of full-softmax attention over a growing key/value cache (the cached
    clean keys/values of all previous frames plus the current pass's own)."""
    import numpy as np
    import torch

    import synth_inputs as SI
    from hybrid_softmax_gated_amd.layer import ARL2Layer, softmax_attention

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = SI.companion(SI.WORKLOADS["long231_480p"])
    B, H, d, L = w.B, w.H, w.d, w.L
    Wd = torch.from_numpy(SI.make_weights(w)).to(dev).to(torch.bfloat16)
    out = torch.empty((B, L, H, d), dtype=torch.bfloat16, device=dev)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]

    def mem():
        free, total = torch.cuda.mem_get_info()
        return torch.cuda.memory_allocated(), total - free

    # untimed warm-up of both paths (first launches, code loading)
    warm = ARL2Layer(B, H, d, L, 0 if w.dtype == SI.BF16 else 1)
    for q in SI.iter_passes_device(w, dev, frames=2):
        warm.forward(q.q, q.k, q.v, Wd, q.alpha, q.beta, out, q.update)
        softmax_attention(q.q, q.k, q.v, out, 0)
    torch.cuda.synchronize()
    del warm
    torch.cuda.empty_cache()

    res = {"workload": w.name, "frames": w.frames, "passes_per_frame": w.passes_per_frame,
           "arl2_ms": [], "arl2_alloc": [], "arl2_used": [],
           "kv_ms": [], "kv_alloc": [], "kv_used": [], "kv_cache_tokens": []}
    # the layer
    layer = ARL2Layer(B, H, d, L, 0 if w.dtype == SI.BF16 else 1)
    cur = []
    for p in SI.iter_passes_device(w, dev):
        cur.append(p)
        if not p.update:
            continue
        torch.cuda.synchronize()
        ev[0].record()
        for q in cur:
            layer.forward(q.q, q.k, q.v, Wd, q.alpha, q.beta, out, q.update)
        ev[1].record()
        torch.cuda.synchronize()
        res["arl2_ms"].append(ev[0].elapsed_time(ev[1]))
        a, u = mem()
        res["arl2_alloc"].append(a)
        res["arl2_used"].append(u)
        cur = []
    del layer
    torch.cuda.empty_cache()
    # The comparator: every pass attends over the cached clean keys/values of
    # all previous frames followed by its own. The cache grows by one frame
    # per frame, in a buffer whose capacity doubles when full (so device
    # memory grows with the frame index while copies stay amortised).
    cap = 1
    kc = torch.empty((B, cap * L, H, d), dtype=torch.bfloat16, device=dev)
    vc = torch.empty_like(kc)
    cur = []
    nf = 0
    for p in SI.iter_passes_device(w, dev):
        cur.append(p)
        if not p.update:
            continue
        if nf + 1 > cap:
            cap *= 2
            k2 = torch.empty((B, cap * L, H, d), dtype=torch.bfloat16, device=dev)
            v2 = torch.empty_like(k2)
            k2[:, :nf * L] = kc[:, :nf * L]
            v2[:, :nf * L] = vc[:, :nf * L]
            kc, vc = k2, v2
            del k2, v2
        lk = (nf + 1) * L
        torch.cuda.synchronize()
        ms = 0.0
        for q in cur:
            kc[:, nf * L:lk] = q.k
            vc[:, nf * L:lk] = q.v
            ev[2].record()
            softmax_attention(q.q, kc[:, :lk], vc[:, :lk], out, 0)
            ev[3].record()
            torch.cuda.synchronize()
            ms += ev[2].elapsed_time(ev[3])
        nf += 1  # the clean pass's keys/values stay in the cache
        res["kv_ms"].append(ms)
        a, u = mem()
        res["kv_alloc"].append(a)
        res["kv_used"].append(u)
        res["kv_cache_tokens"].append(nf * L)
        cur = []
    with open(path, "w") as f:
        json.dump(res, f)
    n = len(res["arl2_ms"])
    pick = [0, 9, 49, 99, n - 1]
    summ = {"metric": "per-frame GPU latency and device memory vs frame index, long horizon "
                      "(231 frames x (1 query-only + 1 clean pass), 12 heads, d=128, L=1560)",
            "frames": n,
            "arl2_ms": {i + 1: round(res["arl2_ms"][i], 4) for i in pick},
            "kv_cache_ms": {i + 1: round(res["kv_ms"][i], 4) for i in pick},
            "arl2_allocated_mb": {i + 1: round(res["arl2_alloc"][i] / 1e6, 3) for i in pick},
            "kv_cache_allocated_mb": {i + 1: round(res["kv_alloc"][i] / 1e6, 3) for i in pick},
            "kv_cache_live_mb": {i + 1: round(res["kv_cache_tokens"][i] * H * d * 4 / 1e6, 3)
                                 for i in pick},
            "speedup_at_last_frame": round(res["kv_ms"][-1] / res["arl2_ms"][-1], 2),
            "cumulative_ms": {"arl2": round(sum(res["arl2_ms"]), 2),
                              "kv_cache": round(sum(res["kv_ms"]), 2)},
            "detail": path}
    print(json.dumps(summ), flush=True)
    return 0


def stack_report(path, frames, layers=30, ratios=(0.0, 0.5, 0.75), pool=4):
    """An attention-only stack: `layers` self-attention layers per pass, of
    which round(ratio * layers) are this layer and the rest full-softmax
    attention over their own key/value cache (the clean keys/values of every
    previous frame, then the pass's own; hybrid_softmax_gated_amd.stack), for
    4 query-only + 1 clean passes per latent frame. Activations are synthetic
    and cycled from a small pool (the work does not depend on the values).
    Per frame: GPU time of all layers and passes (HIP events around the
    frame) and allocated device memory after the frame."""
    import torch

    import synth_inputs as SI
    from hybrid_softmax_gated_amd.stack import AttentionStack

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = SI.scaled(SI.companion(SI.WORKLOADS["stream21_480p"]), frames=pool)
    B, H, d, L = w.B, w.H, w.d, w.L
    npass = w.passes_per_frame
    Wd = torch.from_numpy(SI.make_weights(w)).to(dev).to(torch.bfloat16)
    inputs = list(SI.iter_passes_device(w, dev))  # pool x passes_per_frame
    out = torch.empty((B, L, H, d), dtype=torch.bfloat16, device=dev)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    base_alloc = torch.cuda.memory_allocated()
    res = {"layers": layers, "frames": frames, "passes_per_frame": npass, "runs": {}}
    for ratio in ratios:
        n_arl2 = int(round(ratio * layers))
        stack = AttentionStack(B, H, d, L, layers, n_arl2, device=dev)
        run = {"arl2_layers": n_arl2, "softmax_layers": layers - n_arl2, "ms": [],
               "allocated": []}
        for f in range(frames):
            for c in stack.caches:  # room for this frame's keys/values, outside the timing
                c.reserve(f + 1)
            torch.cuda.synchronize()
            ev[0].record()
            for ps in range(npass):
                for li in range(layers):
                    p = inputs[((f + li) % pool) * npass + ps]
                    stack.forward(li, f, p.q, p.k, p.v, Wd, p.alpha, p.beta, out, p.update)
            ev[1].record()
            torch.cuda.synchronize()
            run["ms"].append(ev[0].elapsed_time(ev[1]))
            run["allocated"].append(torch.cuda.memory_allocated() - base_alloc)
            if f % 25 == 0 or f == frames - 1:
                print(f"stack {int(ratio * 100)}% frame {f + 1}: {run['ms'][-1]:.2f} ms, "
                      f"{run['allocated'][-1] / 1e9:.2f} GB", file=sys.stderr, flush=True)
        res["runs"][f"{int(ratio * 100)}%"] = run
        del stack
        torch.cuda.empty_cache()
    with open(path, "w") as fh:
        json.dump(res, fh)
    summ = {"metric": f"attention-only stack of {layers} layers, per-frame GPU ms and allocated "
                      f"GB vs latent frame ({npass - 1} query-only + 1 clean passes, 12 heads, "
                      f"d=128, L=1560)", "frames": frames}
    for k, r in res["runs"].items():
        pick = sorted({0, 20, 80, 230, frames - 1} & set(range(frames)))
        summ[k] = {"ms": {i + 1: round(r["ms"][i], 3) for i in pick},
                   "allocated_gb": {i + 1: round(r["allocated"][i] / 1e9, 3) for i in pick},
                   "total_s": round(sum(r["ms"]) / 1e3, 3)}
    print(json.dumps(summ), flush=True)
    return 0


def gate_projection_leg(w, dev, stream, steps, repeat):
    """Per-call GPU time of the gate projections (alpha and beta from the layer
    input x [B][L][D], D = H*d, weights [H][D]) on the workload's shape,
    against the HBM roofline: x, both weights and the gates are moved once.

    The call is two short launches; issued from the host one by one, they
    finish faster than the host enqueues them, so the time is taken from a
    HIP graph of `repeat` calls replayed `steps` times (events on the
    replay stream), and every replay's gates are checked against the eager
    call's."""
    import torch

    import synth_inputs as SI
    from hybrid_softmax_gated_amd import binding as Bd
    from hybrid_softmax_gated_amd.layer import gate_projections

    B, L, D, H = w.B, w.L, w.H * w.d, w.H
    x, Wa, Wb = (torch.from_numpy(t).to(dev).to(torch.bfloat16)
                 for t in SI.make_gate_inputs(B, L, D, H, SI.BF16, w.seed))
    alpha, beta, ws = gate_projections(x, Wa, Wb, Bd.ARL2_BF16, stream=stream)
    torch.cuda.synchronize()
    a_ref, b_ref = alpha.clone(), beta.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        cap = torch.cuda.current_stream()
        for _ in range(repeat):
            gate_projections(x, Wa, Wb, Bd.ARL2_BF16, alpha, beta, ws, cap)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ms = 0.0
    for _ in range(steps):
        alpha.zero_()
        beta.zero_()
        torch.cuda.synchronize()
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        ms += e0.elapsed_time(e1)
        assert torch.equal(alpha, a_ref) and torch.equal(beta, b_ref), "graph replay differs"
    us = 1000.0 * ms / (steps * repeat)
    nbytes = B * L * D * 2 + 2 * H * D * 2 + B * L * H * 4 + B * H * 4
    gbs = nbytes / (us * 1e-6) / 1e9
    return {"bound": "hbm", "avg_call_us": round(us, 2), "bytes_per_call": nbytes,
            "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(gbs / PEAK_HBM_GBS, 4),
            "shape": f"x [{B}][{L}][{D}] bf16, Wa/Wb [{H}][{D}]",
            "timing": f"HIP graph of {repeat} calls (2 launches each), {steps} replays"}


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--device-warmup-ms", type=float, default=200.0,
                    help="before the --warmup frames, run whole frames untimed for this much "
                         "wall time: from idle the GPU's clocks take about 40 ms of load to reach "
                         "their steady state, which a short timed region would otherwise measure")
    ap.add_argument("--workload", default="stream21_480p",
                    choices=["frame_step_480p", "stream21_480p", "batched720p"])
    ap.add_argument("--gate", default="headwise", choices=["headwise", "elementwise"],
                    help="forget gate: one scalar per head (the method's) or one value per "
                         "d_k row (the ablation's)")
    ap.add_argument("--access", default="frame", choices=["frame", "token"],
                    help="state access: frame-level (the method's) or token-level (the "
                         "ablation's: tokens write the state in turn, each reading it after "
                         "its own write)")
    ap.add_argument("--stack-report", metavar="PATH", default="",
                    help="instead of the throughput line: an attention-only stack of 30 layers "
                         "in which 0, 50 and 75 %% of the softmax KV-cache layers are replaced by "
                         "this layer, run over --stack-frames latent frames of 4 query-only + 1 "
                         "clean passes; writes per-frame GPU time and device memory to PATH")
    ap.add_argument("--stack-frames", type=int, default=252)
    ap.add_argument("--per-frame-report", metavar="PATH", default="",
                    help="instead of the throughput line: run the 231-frame long-horizon "
                         "schedule through the layer and through full-softmax attention over a "
                         "key/value cache that grows by one frame per frame, and write per-frame "
                         "GPU latency and device memory of both to PATH (JSON)")
    ap.add_argument("--profile-steps", type=int, default=100)
    ap.add_argument("--profile-repeat", type=int, default=10,
                    help="back-to-back launches of each idempotent kernel per event pair "
                         "in the per-kernel timing leg")
    ap.add_argument("--gate-projections-only", action="store_true",
                    help="only time the gate projections on the workload's shape and print "
                         "their JSON object")
    ap.add_argument("--graph", action="store_true",
                    help="capture the cycle of distinct frames into one HIP graph and time its "
                         "replays instead of eager calls")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="only copy a buffer of this many MiB 10 times (scales the HBM byte "
                         "counters of a profiler run) and exit")
    args = ap.parse_args()

    if args.calibrate_copy_mib:
        import torch
        n = args.calibrate_copy_mib << 20
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(10):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copied_bytes_per_launch": n, "launches": 10}))
        return 0
    if args.gpus != 1:
        print(f"bench.py: the benchmark measures one GPU; --gpus {args.gpus} is not supported "
              "(the layer would shard by stream and head, with no exchange between GPUs)",
              file=sys.stderr)
        return 2
    if args.per_frame_report:
        return per_frame_report(args.per_frame_report)
    if args.stack_report:
        return stack_report(args.stack_report, args.stack_frames)

    import numpy as np
    import torch

    import synth_inputs as SI
    from hybrid_softmax_gated_amd import binding as Bd

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = SI.scaled(SI.companion(SI.WORKLOADS[args.workload]), gate=args.gate)
    if args.gate != "headwise":
        w = SI.scaled(w, name=f"{w.name}_{args.gate}_gate")
    if args.access == "token":
        if args.gate != "headwise":
            print("bench.py: token-level access takes the headwise gate", file=sys.stderr)
            return 2
        w = SI.scaled(w, name=f"{w.name}_token_level")
    B, H, d, L = w.B, w.H, w.d, w.L

    if args.gate_projections_only:
        leg = gate_projection_leg(w, dev, torch.cuda.current_stream(), 20, 50)
        print(json.dumps({"workload": w.name, "gate_projections": leg}), flush=True)
        return 0

    stream = torch.cuda.current_stream()
    main_leg = time_schedule(w, dev, stream, args.steps, args.warmup, args.access,
                             graph=args.graph, profile_steps=args.profile_steps,
                             profile_repeat=args.profile_repeat,
                             device_warmup_ms=args.device_warmup_ms)
    if main_leg is None:
        return 2
    fps = main_leg["fps"]
    kern_us = main_leg["kernels_us"]

    # The single 480p frame step's 1 + 1 schedule, a shorter timed leg.
    extra = None
    if args.workload != "frame_step_480p" and args.access == "frame" and args.gate == "headwise":
        w11 = SI.companion(SI.WORKLOADS["frame_step_480p"])
        leg = time_schedule(w11, dev, stream, max(200, args.steps // 2), args.warmup, "frame",
                            profile_steps=max(20, args.profile_steps // 2), profile_repeat=1,
                            device_warmup_ms=min(50.0, args.device_warmup_ms))
        fa11, fb11, fc11 = flops(w11.B, w11.H, w11.d, w11.L)
        extra = {"workload": w11.name, "passes_per_frame": "1 query-only + 1 clean",
                 "value": round(leg["fps"], 2), "unit": "frames/s",
                 "ms_per_step": round(1000.0 / leg["fps"], 5),
                 "tflops": round((2 * (fa11 + fb11) + fc11) * leg["fps"] / 1e12, 2),
                 "kernels_us": {k: round(v, 2) for k, v in leg["kernels_us"].items()},
                 "frame_latency": leg["frame_latency"]}

    gate_leg = gate_projection_leg(w, dev, stream, 20, 50)
    mfma_loop = max(Bd.arl2_profile_mfma_peak(4096, stream) for _ in range(3))

    fa, fb, fc = flops(B, H, d, L)
    passes = w.passes_per_frame
    frame_flops = passes * (fa + fb) + fc
    tflops = frame_flops * fps / 1e12
    digest = source_digest("attn.hip", "arl2_device.h", "delta_chunk.h")
    res = {
        "metric": METRIC, "value": round(fps, 2), "unit": "frames/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup,
        "device_warmup": {"ms": args.device_warmup_ms, "frames": main_leg["device_warmup_frames"],
                          "what": "whole frames of the same workload, untimed, before the "
                                  "warm-up frames, so that the GPU's clocks have left their "
                                  "idle ramp"},
        "ms_per_step": round(1000.0 * main_leg["wall"] / args.steps, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "B": B, "H": H, "d": d, "L": L,
                   "launch": "HIP graph replay" if args.graph else "eager",
                   "passes_per_frame": f"{w.noisy_passes} query-only + 1 clean",
                   "distinct_frames_cycled": NUM_DISTINCT_FRAMES},
        "tflops": round(tflops, 2), "frac_bf16_peak": round(tflops / PEAK_BF16_TFLOPS, 4),
        "gflop_per_frame": round(frame_flops / 1e9, 3),
        "event_ms_per_step": round(main_leg["event_ms"] / args.steps, 5),
        "frame_latency": main_leg["frame_latency"],
        "kernels_us": {k: round(v, 2) for k, v in kern_us.items()},
        "kernels_us_warm": {k: round(v, 2) for k, v in main_leg["kernels_us_warm"].items()},
        "kernels_timing": "kernels_us: in sequence, HIP events from the kernels' own start and "
                          f"end (repeat 1, {args.profile_steps} frames); kernels_us_warm: each "
                          f"idempotent launch {args.profile_repeat} times back to back between "
                          "two event markers",
    }
    if d == 128 and w.dtype == SI.BF16 and args.access == "frame" and "attn_partial" in kern_us:
        att_us = kern_us["attn_partial"]
        att_tflops = fa / (att_us * 1e-6) / 1e12
        traffic = measured_traffic("attn_partial", args.workload, digest)
        alg_bytes = method_bytes(B, H, d, L)["attn_partial"]["method"]
        res["roofline"] = {
            "bound": "mfma", "achieved": round(att_tflops, 2), "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s", "frac": round(att_tflops / PEAK_BF16_TFLOPS, 4),
            "traffic": traffic, "kernel": "attn_partial (query-only pass, first launch)",
            "per_launch": f"4*B*H*L^2*d = {fa / 1e9:.3f} GFLOP (one pass, B={B} H={H} L={L} "
                          f"d={d})",
            "avg_launch_us": round(att_us, 2),
            "timing": "in sequence: HIP events from the kernel's own start and end",
            "warm_repeat_us": round(main_leg["kernels_us_warm"].get("attn_partial", 0.0), 2),
            "frac_of_measured_mfma_loop": round(att_tflops / mfma_loop, 4),
            "traffic_ratio": round(traffic / alg_bytes, 3) if traffic else None,
            "algorithmic_bytes": alg_bytes}
        ctr = launch_counters(args.workload)
        if "attn_delta" in kern_us:
            dt = kern_us["attn_delta"] - att_us
            res["delta_update"] = {
                "bound": "mfma", "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "per_clean_pass": f"8*B*H*L*d^2 = {fc / 1e9:.3f} GFLOP algorithmic; the split-bf16 "
                                  f"products execute {2 * fc / 1e9:.3f} GFLOP",
                "added_us": round(dt, 2),
                "achieved": round(fc / (dt * 1e-6) / 1e12, 2) if dt > 0 else None,
                "frac": round(fc / (dt * 1e-6) / 1e12 / PEAK_BF16_TFLOPS, 4) if dt > 0 else None,
                "executed_tflops": round(2 * fc / (dt * 1e-6) / 1e12, 2) if dt > 0 else None,
                "timing": "in sequence: the clean pass's first launch (attention + delta chunks) "
                          "minus the query-only pass's (attention alone); the two launches run the "
                          "attention in 4- and 8-wavefront workgroups, which at 480p measure "
                          "within 1 % of each other alone"}
            if "attn_delta" in ctr and "attn_partial" in ctr:
                res["delta_update"]["mfma_util_pct"] = {
                    "attn_delta": ctr["attn_delta"]["mfma_util_pct"],
                    "attn_partial": ctr["attn_partial"]["mfma_util_pct"],
                    "pure_mfma_loop": ctr["mfma_loop_util_pct"],
                    "source": "rocprofv3 MfmaUtil, committed counter summary of this workload"}
        epi = {}
        mb = method_bytes(B, H, d, L)
        for name in ("combine", "combine_apply"):
            if name in kern_us:
                nbytes = mb[name]["method"]
                gbs = nbytes / (kern_us[name] * 1e-6) / 1e9
                tr = ctr.get(name, {}).get("bytes_per_launch")
                epi[name] = {"bound": "hbm", "bytes": int(nbytes),
                             "scratch_bytes": int(mb[name]["scratch"]),
                             "avg_launch_us": round(kern_us[name], 2), "achieved": round(gbs, 1),
                             "peak": PEAK_HBM_GBS, "unit": "GB/s",
                             "frac": round(gbs / PEAK_HBM_GBS, 4),
                             "traffic": tr,
                             "traffic_ratio": round(tr / nbytes, 3) if tr else None}
        res["epilogues"] = epi
    res["mfma_loop_peak_tflops"] = round(mfma_loop, 1)
    if extra is not None:
        res["frame_step_1p1"] = extra
    res["gate_projections"] = gate_leg
    if not args.no_cpu_baseline:
        host = []
        for fr in main_leg["frames"][:2]:
            host.append([{"q": p.q.float().cpu().numpy(), "k": p.k.float().cpu().numpy(),
                          "v": p.v.float().cpu().numpy(), "alpha": p.alpha.cpu().numpy(),
                          "beta": p.beta.cpu().numpy(), "update": p.update} for p in fr])
        W = SI.make_weights(w)
        res["cpu_baseline"] = cpu_baseline(host, W, w, access=args.access)
    print(json.dumps(res), flush=True)
    return 0


def time_schedule(w, dev, stream, steps, warmup, access, graph=False, profile_steps=100,
                  profile_repeat=10, device_warmup_ms=0.0):
    """Draw NUM_DISTINCT_FRAMES frames of workload w on the GPU, then: run
    whole frames untimed for `device_warmup_ms` of wall time (the GPU's clocks
    ramp up from idle over the first tens of milliseconds of load), warm up
    `warmup` frames, time `steps` frames (cycled) between two
    synchronizations, time 200 frames one by one with HIP events, and take
    per-kernel times in sequence (repeat 1) and, if profile_repeat > 1, warm
    (repeated back to back)."""
    import torch

    import synth_inputs as SI
    from hybrid_softmax_gated_amd import binding as Bd
    from hybrid_softmax_gated_amd.layer import ARL2Layer

    B, H, d, L = w.B, w.H, w.d, w.L
    Wd = torch.from_numpy(SI.make_weights(w)).to(dev).to(torch.bfloat16)
    frames, cur = [], []
    for p in SI.iter_passes_device(w, dev, frames=NUM_DISTINCT_FRAMES):
        cur.append(p)
        if p.update:
            frames.append(cur)
            cur = []
    layer = ARL2Layer(B, H, d, L, Bd.ARL2_BF16)
    out = torch.empty((B, L, H, d), dtype=torch.bfloat16, device=dev)

    def step(i, s=stream):
        for p in frames[i % len(frames)]:
            if access == "token":
                layer.forward_token_level(p.q, p.k, p.v, Wd, p.alpha, p.beta, out, p.update, s)
            else:
                layer.forward(p.q, p.k, p.v, Wd, p.alpha, p.beta, out, p.update, s, gate=w.gate)

    # Device warm-up: full frames, untimed, until the wall-time budget is
    # spent (synchronising every few frames so the host does not run ahead).
    n_dev_warm = 0
    t_end = time.perf_counter() + device_warmup_ms / 1000.0
    while time.perf_counter() < t_end:
        for _ in range(8):
            step(n_dev_warm)
            n_dev_warm += 1
        torch.cuda.synchronize()

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()

    g = None
    if graph:
        # The cycle of distinct frames as one HIP graph, replayed steps / cycle times.
        if steps % len(frames):
            print(f"bench.py: --graph needs --steps to be a multiple of {len(frames)}",
                  file=sys.stderr)
            return None
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            cap = torch.cuda.current_stream()
            for i in range(len(frames)):
                step(i, cap)
        torch.cuda.synchronize()
        g.replay()          # one untimed replay
        torch.cuda.synchronize()

    # ---- timed region (single process: the barrier is the synchronize)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    if g is not None:
        for _ in range(steps // len(frames)):
            g.replay()
    else:
        for i in range(steps):
            step(i)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    event_ms = ev0.elapsed_time(ev1)
    assert torch.isfinite(layer.S).all(), "state went non-finite during the benchmark"

    # ---- per-frame latency: HIP events around each frame (eager), after 10
    # warm-up frames; the median of 200 frames
    for i in range(10):
        step(i)
    fev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(200)]
    for i, (e0, e1) in enumerate(fev):
        e0.record(stream)
        step(i)
        e1.record(stream)
    torch.cuda.synchronize()
    per_frame = sorted(e0.elapsed_time(e1) for e0, e1 in fev)
    frame_latency = {"median_ms": round(per_frame[len(per_frame) // 2], 5),
                     "p10_ms": round(per_frame[len(per_frame) // 10], 5),
                     "p90_ms": round(per_frame[(9 * len(per_frame)) // 10], 5),
                     "frames": len(per_frame), "warmup": 10,
                     "timing": "HIP events around each frame's passes, eager launches"}

    def kernel_times(repeat):
        Bd.arl2_profile_reset()
        Bd.arl2_profile_enable(True, repeat)
        for i in range(profile_steps):
            step(i)
        torch.cuda.synchronize()
        rep = Bd.arl2_profile_report()
        Bd.arl2_profile_enable(False)
        return {k: 1000.0 * ms / n for k, (n, ms) in rep.items() if n}

    kern_us = kernel_times(1)
    kern_warm = kernel_times(profile_repeat) if profile_repeat > 1 else {}
    return {"fps": steps / wall, "wall": wall, "event_ms": event_ms, "frames": frames,
            "frame_latency": frame_latency, "kernels_us": kern_us, "kernels_us_warm": kern_warm,
            "device_warmup_frames": n_dev_warm}


if __name__ == "__main__":
    sys.exit(main())
