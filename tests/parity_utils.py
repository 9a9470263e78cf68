"""Helpers shared by the GPU parity tests (not a test module)."""
from __future__ import annotations

import contextlib
import os
import time

import numpy as np

import oracle as O
import synth_inputs as SI

# Tolerances of the parity contract: outputs (max |gpu - ref| / max |ref| per
# output tensor per pass) and state (the same per (stream, head)).
TOL_OUT = {SI.BF16: 2e-2, SI.F32: 1e-4}
TOL_S = 1e-3


def torch_mod():
    import torch
    return torch


def device():
    torch = torch_mod()
    assert torch.cuda.is_available(), "GPU tests need a ROCm GPU (torch.cuda.is_available())"
    return torch.device("cuda:0")


def to_dev(x: np.ndarray, dtype: str):
    """Upload float32 values (bf16-exact for bf16 workloads) in the io dtype."""
    torch = torch_mod()
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(device())
    return t.to(SI.torch_dtype(dtype)) if dtype == SI.BF16 else t


def to_host(t) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def rel_max_err(got: np.ndarray, ref: np.ndarray) -> float:
    den = float(np.max(np.abs(ref)))
    num = float(np.max(np.abs(got - ref)))
    if den == 0.0:
        return num
    return num / den


def state_err(S_gpu: np.ndarray, S_ref: np.ndarray) -> float:
    """Worst per-(stream, head) max-norm relative error of the state."""
    B, H = S_ref.shape[:2]
    return max(rel_max_err(S_gpu[b, h], S_ref[b, h]) for b in range(B) for h in range(H))


def out_err_per_head(got: np.ndarray, ref: np.ndarray) -> float:
    """Worst per-(stream, head) max-norm relative error of an output [B][L][H][d]."""
    B, _, H, _ = ref.shape
    return max(rel_max_err(got[b, :, h], ref[b, :, h]) for b in range(B) for h in range(H))


def oracle_state_update(S: np.ndarray, k: np.ndarray, v: np.ndarray, W: np.ndarray,
                        alpha: np.ndarray, beta: np.ndarray) -> None:
    """Advance the float64 oracle state S [B][H][d][d] in place by one clean
    pass (only the state part of the oracle's frame step)."""
    B, L, H, d = k.shape
    for b in range(B):
        for h in range(H):
            Kp = O.l2_normalize_rows(O.feature_map(k[b, :, h], W[1, h]))
            Vp = O.feature_map(v[b, :, h], W[2, h])
            S[b, h] = O.delta_update(S[b, h], Kp, Vp, alpha[b, h], beta[b, :, h])


def oracle_rows(q, k, v, W, S, rows_per_head: np.ndarray):
    """Oracle output for sampled rows of every (stream, head):
    returns [B][R][H][d] for the row indices ``rows_per_head``."""
    B, L, H, d = q.shape
    out = np.empty((B, len(rows_per_head), H, d))
    for b in range(B):
        for h in range(H):
            out[b, :, h] = O.output_rows(q[b, :, h], k[b, :, h], v[b, :, h], W[0, h], S[b, h],
                                         rows_per_head)
    return out


def sample_rows(L: int, n: int, seed: int) -> np.ndarray:
    """Sorted row indices: the first, the last, the last full tile's edges and
    random rows."""
    r = np.random.default_rng(seed)
    fixed = {0, L - 1, min(L - 1, 127), min(L - 1, 128), (L - 1) // 128 * 128}
    extra = r.choice(L, size=min(L, n), replace=False)
    return np.array(sorted(fixed | set(int(x) for x in extra)))


# Host wall time the float64 oracle spends per workload in the parity tests,
# with the threads it ran on; the session summary prints it (conftest.py).
ORACLE_SECONDS: dict = {}


@contextlib.contextmanager
def oracle_clock(workload: str):
    t0 = time.perf_counter()
    try:
        yield
    finally:
        ORACLE_SECONDS[workload] = ORACLE_SECONDS.get(workload, 0.0) + time.perf_counter() - t0


def oracle_threads() -> str:
    try:
        from threadpoolctl import threadpool_info
        n = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # threadpoolctl is optional
        n = None
    return f"BLAS threads {n}, os.cpu_count() {os.cpu_count()}"
