"""ctypes binding of libarl2 (include/arl2.h).

Argument marshalling only: every function below forwards to the C entry
point of the same name. Tensor arguments may be raw device addresses (int)
or any object with ``data_ptr()`` (a torch tensor); ``stream`` may be a
hipStream_t address (int), an object with ``cuda_stream`` (a torch stream)
or None for torch's current stream on the current device (the default
stream when torch is not loaded).

The library is loaded from this package's directory; if it is missing the
import of this module raises, so no caller can silently fall back to other
code.
"""
from __future__ import annotations

import ctypes
import os
import sys

ARL2_OK = 0
ARL2_ERR_INVALID_ARG = 1
ARL2_ERR_UNSUPPORTED = 2
ARL2_ERR_HIP = 3
ARL2_BF16 = 0
ARL2_F32 = 1
ARL2_GATE_HEADWISE = 0
ARL2_GATE_ELEMENTWISE = 1

# The in-tree library; ARL2_LIBRARY may name another build of the same ABI
# (for comparing kernel variants).
LIB_PATH = os.environ.get("ARL2_LIBRARY") or os.path.join(
    os.path.dirname(os.path.abspath(__file__)), "libarl2.so")


class arl2_state(ctypes.Structure):
    """Mirror of the C ``arl2_state`` descriptor."""

    _fields_ = [
        ("B", ctypes.c_int32),
        ("H", ctypes.c_int32),
        ("d", ctypes.c_int32),
        ("L", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("magic", ctypes.c_int32),
        ("S", ctypes.c_void_p),
        ("ws", ctypes.c_void_p),
        ("ws_bytes", ctypes.c_size_t),
    ]


class ARL2Error(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"libarl2.so is not built ({LIB_PATH}); run "
                          "`python -m hybrid_softmax_gated_amd.build` or __graft_entry__.build()")
    lib = ctypes.CDLL(LIB_PATH)
    P, I, Z = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    sig = {
        "arl2_version": (I, []),
        "arl2_status_string": (ctypes.c_char_p, [I]),
        "arl2_last_error": (ctypes.c_char_p, []),
        "arl2_workspace_bytes": (Z, [I, I, I, I, I]),
        "arl2_state_init": (I, [ctypes.POINTER(arl2_state), I, I, I, I, I, P, P, Z, P]),
        "arl2_state_reset": (I, [ctypes.POINTER(arl2_state), P, P]),
        "arl2_frame_forward": (I, [P, P, P, P, ctypes.POINTER(arl2_state), P, P, P, I, P]),
        "arl2_frame_forward_gated": (I, [P, P, P, P, ctypes.POINTER(arl2_state), P, I, P, P, I,
                                         P]),
        "arl2_frame_forward_noalloc": (I, [P, P, P, P, ctypes.POINTER(arl2_state), P, P, P, I,
                                           P]),
        "arl2_token_level_workspace_bytes": (Z, [I, I, I, I, I]),
        "arl2_frame_forward_token_level": (I, [P, P, P, P, ctypes.POINTER(arl2_state), P, P, P, I,
                                               P, Z, P]),
        "arl2_softmax_attention_workspace_bytes": (Z, [I, I, I, I, I, I]),
        "arl2_softmax_attention": (I, [P, P, P, I, I, I, I, I, I, P, P, Z, P]),
        "arl2_gate_projections_workspace_bytes": (Z, [I, I, I, I, I]),
        "arl2_gate_projections": (I, [P, P, P, I, I, I, I, I, P, P, P, Z, P]),
        "arl2_profile_enable": (I, [I, I]),
        "arl2_profile_report": (I, [ctypes.c_char_p, Z]),
        "arl2_profile_reset": (None, []),
        "arl2_profile_mfma_peak": (I, [I, ctypes.POINTER(ctypes.c_double), P]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


_lib = _load()

EXPORTED = ("arl2_version", "arl2_status_string", "arl2_last_error", "arl2_workspace_bytes",
            "arl2_state_init", "arl2_state_reset", "arl2_frame_forward", "arl2_frame_forward_gated",
            "arl2_frame_forward_noalloc",
            "arl2_softmax_attention_workspace_bytes", "arl2_softmax_attention",
            "arl2_gate_projections_workspace_bytes", "arl2_gate_projections",
            "arl2_token_level_workspace_bytes", "arl2_frame_forward_token_level",
            "arl2_profile_enable", "arl2_profile_report", "arl2_profile_reset",
            "arl2_profile_mfma_peak")


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if hasattr(x, "is_contiguous") and not x.is_contiguous():
        raise ValueError("libarl2 takes contiguous tensors (call .contiguous() first)")
    return int(x.data_ptr())


def _stream(s):
    if s is None:
        torch = sys.modules.get("torch")
        if torch is not None and torch.cuda.is_available() and torch.cuda.is_initialized():
            return int(torch.cuda.current_stream().cuda_stream)
        return None
    if isinstance(s, int):
        return s
    return int(s.cuda_stream)


def _check(status: int) -> None:
    if status != ARL2_OK:
        msg = _lib.arl2_last_error().decode()
        raise ARL2Error(status, f"{_lib.arl2_status_string(status).decode()}: {msg}")


def arl2_version() -> int:
    return int(_lib.arl2_version())


def arl2_status_string(status: int) -> str:
    return _lib.arl2_status_string(status).decode()


def arl2_last_error() -> str:
    return _lib.arl2_last_error().decode()


def arl2_workspace_bytes(B: int, H: int, d: int, L: int, dtype: int) -> int:
    return int(_lib.arl2_workspace_bytes(B, H, d, L, dtype))


def arl2_state_init(st: arl2_state, B: int, H: int, d: int, L: int, dtype: int, S, ws,
                    ws_bytes: int, stream=None) -> None:
    _check(_lib.arl2_state_init(ctypes.byref(st), B, H, d, L, dtype, _ptr(S), _ptr(ws),
                                ws_bytes, _stream(stream)))


def arl2_state_reset(st: arl2_state, S0=None, stream=None) -> None:
    _check(_lib.arl2_state_reset(ctypes.byref(st), _ptr(S0), _stream(stream)))


def arl2_frame_forward(q, k, v, Wphi, st: arl2_state, alpha, beta, out, update_flag: int,
                       stream=None) -> None:
    _check(_lib.arl2_frame_forward(_ptr(q), _ptr(k), _ptr(v), _ptr(Wphi), ctypes.byref(st),
                                   _ptr(alpha), _ptr(beta), _ptr(out), update_flag,
                                   _stream(stream)))


def arl2_frame_forward_gated(q, k, v, Wphi, st: arl2_state, alpha, gate: int, beta, out,
                             update_flag: int, stream=None) -> None:
    _check(_lib.arl2_frame_forward_gated(_ptr(q), _ptr(k), _ptr(v), _ptr(Wphi), ctypes.byref(st),
                                         _ptr(alpha), gate, _ptr(beta), _ptr(out), update_flag,
                                         _stream(stream)))


# Bytes of scratch the no-allocation pass holds per device (include/arl2.h).
ARL2_NOALLOC_SCRATCH_BYTES = 32 << 20


def arl2_frame_forward_noalloc(q, k, v, Wphi, st: arl2_state, alpha, beta, out, update_flag: int,
                               stream=None) -> None:
    _check(_lib.arl2_frame_forward_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(Wphi),
                                           ctypes.byref(st), _ptr(alpha), _ptr(beta), _ptr(out),
                                           update_flag, _stream(stream)))


def arl2_token_level_workspace_bytes(B: int, H: int, d: int, L: int, dtype: int) -> int:
    return int(_lib.arl2_token_level_workspace_bytes(B, H, d, L, dtype))


def arl2_frame_forward_token_level(q, k, v, Wphi, st: arl2_state, alpha, beta, out,
                                   update_flag: int, tl_ws, tl_ws_bytes: int, stream=None) -> None:
    _check(_lib.arl2_frame_forward_token_level(_ptr(q), _ptr(k), _ptr(v), _ptr(Wphi),
                                               ctypes.byref(st), _ptr(alpha), _ptr(beta),
                                               _ptr(out), update_flag, _ptr(tl_ws), tl_ws_bytes,
                                               _stream(stream)))


def arl2_softmax_attention_workspace_bytes(B: int, H: int, d: int, Lq: int, Lk: int,
                                           dtype: int) -> int:
    return int(_lib.arl2_softmax_attention_workspace_bytes(B, H, d, Lq, Lk, dtype))


def arl2_softmax_attention(q, kc, vc, B: int, H: int, d: int, Lq: int, Lk: int, dtype: int, out,
                           ws, ws_bytes: int, stream=None) -> None:
    _check(_lib.arl2_softmax_attention(_ptr(q), _ptr(kc), _ptr(vc), B, H, d, Lq, Lk, dtype,
                                       _ptr(out), _ptr(ws), ws_bytes, _stream(stream)))


def arl2_gate_projections_workspace_bytes(B: int, L: int, D: int, H: int, dtype: int) -> int:
    return int(_lib.arl2_gate_projections_workspace_bytes(B, L, D, H, dtype))


def arl2_gate_projections(x, Wa, Wb, B: int, L: int, D: int, H: int, dtype: int, alpha, beta, ws,
                          ws_bytes: int, stream=None) -> None:
    _check(_lib.arl2_gate_projections(_ptr(x), _ptr(Wa), _ptr(Wb), B, L, D, H, dtype, _ptr(alpha),
                                      _ptr(beta), _ptr(ws), ws_bytes, _stream(stream)))


def arl2_profile_enable(on: bool, repeat: int = 1) -> None:
    _check(_lib.arl2_profile_enable(1 if on else 0, int(repeat)))


def arl2_profile_reset() -> None:
    _lib.arl2_profile_reset()


def arl2_profile_mfma_peak(iters: int = 4096, stream=None) -> float:
    """Sustained bf16 MFMA rate of the current device in TFLOP/s (a pure MFMA loop)."""
    out = ctypes.c_double(0.0)
    _check(_lib.arl2_profile_mfma_peak(int(iters), ctypes.byref(out), _stream(stream)))
    return out.value


def arl2_profile_report() -> dict:
    """{kernel name: (launches, total_ms)} for the launches timed so far."""
    buf = ctypes.create_string_buffer(1 << 16)
    _check(_lib.arl2_profile_report(buf, len(buf)))
    res = {}
    for line in buf.value.decode().splitlines():
        name, n, ms = line.split()
        res[name] = (int(n), float(ms))
    return res
