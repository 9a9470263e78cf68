"""The C ABI without a GPU: the library loads, exports exactly what
include/arl2.h declares, and rejects bad arguments before touching HIP.

No call here reaches a kernel: every case fails validation, which runs
before anything is enqueued. Fake device addresses are plain integers that
are never dereferenced.
"""
import ctypes
import os
import re
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "arl2.h")



@pytest.fixture(scope="module")
def B():
    from hybrid_softmax_gated_amd import binding
    return binding


def _declared():
    text = open(HEADER).read()
    return set(re.findall(r"ARL2_API\s+[\w\s\*]*?\b(arl2_\w+)\s*\(", text))


def test_header_declares_the_boundary():
    names = _declared()
    assert {"arl2_state_init", "arl2_state_reset", "arl2_frame_forward",
            "arl2_frame_forward_gated", "arl2_workspace_bytes"} <= names
    assert len(names) == 19


def test_library_exports_every_declared_symbol(B):
    out = subprocess.run(["nm", "-D", "--defined-only", B.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {ln.split()[-1] for ln in out.splitlines() if " T " in ln}
    assert _declared() <= exported
    # nothing else with the public prefix leaks out
    assert {e for e in exported if e.startswith("arl2_")} == _declared()
    assert set(B.EXPORTED) == _declared()


def test_profile_report_without_launches(B):
    B.arl2_profile_reset()
    assert B.arl2_profile_report() == {}
    B.arl2_profile_enable(False)
    for bad in (0, -1, 1001):
        with pytest.raises(B.ARL2Error, match="repeat"):
            B.arl2_profile_enable(True, bad)
    B.arl2_profile_enable(False, 1)


def test_mfma_peak_rejects_bad_arguments_before_touching_the_device(B):
    for bad in (0, -5, (1 << 20) + 1):
        with pytest.raises(B.ARL2Error, match="iters"):
            B.arl2_profile_mfma_peak(bad)
    assert B._lib.arl2_profile_mfma_peak(16, None, None) == B.ARL2_ERR_INVALID_ARG
    assert "tflops" in B.arl2_last_error()


def test_version_and_status_strings(B):
    assert B.arl2_version() == 1
    assert B.arl2_status_string(0) == "ok"
    assert B.arl2_status_string(1) == "invalid argument"
    assert B.arl2_status_string(2) == "unsupported"
    assert B.arl2_status_string(3) == "HIP runtime error"
    assert B.arl2_status_string(99) == "unknown status"


def test_state_struct_layout_matches_c(B):
    assert ctypes.sizeof(B.arl2_state) == 6 * 4 + 3 * 8
    assert B.arl2_state.S.offset == 24 and B.arl2_state.ws_bytes.offset == 40


def test_workspace_bytes(B):
    n = B.arl2_workspace_bytes(1, 12, 128, 1560, B.ARL2_BF16)
    assert n > 0 and n % 256 == 0
    # independent of the number of frames by construction; grows with L
    assert B.arl2_workspace_bytes(1, 12, 128, 3600, B.ARL2_BF16) > n
    assert B.arl2_workspace_bytes(1, 1, 16, 64, B.ARL2_F32) > 0
    for bad in [(0, 12, 128, 1560, 0), (1, 0, 128, 1560, 0), (1, 12, 64, 1560, 0),
                (1, 12, 128, 0, 0), (1, 12, 128, 1560, 7), (1, 12, 128, (1 << 20) + 1, 0)]:
        assert B.arl2_workspace_bytes(*bad) == 0


@pytest.mark.parametrize("Bn,H,L", [(1, 12, 1560), (4, 12, 3600), (2, 3, 200), (3, 1, 1000),
                                    (1, 1, 64), (1, 2, 130), (8, 16, 777)])
def test_bench_epilogue_bytes_follow_the_library_plan(B, Bn, H, L):
    """bench.py reports the design's scratch bytes with its own copy of the
    attention plan; the library's workspace (partials, then the delta
    contributions, then the bf16 copy of the state, each 256-byte aligned)
    must hold exactly those bytes."""
    import bench

    def al(x):
        return (x + 255) // 256 * 256

    o_bytes, ml_bytes, ds, s16 = bench.workspace_parts(Bn, H, 128, L)
    assert B.arl2_workspace_bytes(Bn, H, 128, L, B.ARL2_BF16) == (al(o_bytes) + al(ml_bytes) +
                                                                  al(ds) + al(s16))


FAKE_S = 0x7F0000000000
FAKE_WS = 0x7F1000000000


def _code(fn, *a):
    from hybrid_softmax_gated_amd.binding import ARL2Error
    with pytest.raises(ARL2Error) as ei:
        fn(*a)
    return ei.value.status, str(ei.value)


def test_state_init_validation(B):
    st = B.arl2_state()
    ws = B.arl2_workspace_bytes(1, 2, 128, 100, B.ARL2_BF16)
    assert _code(B.arl2_state_init, st, 1, 2, 64, 100, 0, FAKE_S, FAKE_WS, ws)[0] == B.ARL2_ERR_UNSUPPORTED
    assert _code(B.arl2_state_init, st, 0, 2, 128, 100, 0, FAKE_S, FAKE_WS, ws)[0] == B.ARL2_ERR_INVALID_ARG
    assert _code(B.arl2_state_init, st, 1, 2, 128, 100, 5, FAKE_S, FAKE_WS, ws)[0] == B.ARL2_ERR_INVALID_ARG
    assert _code(B.arl2_state_init, st, 1, 2, 128, 100, 0, None, FAKE_WS, ws)[0] == B.ARL2_ERR_INVALID_ARG
    assert _code(B.arl2_state_init, st, 1, 2, 128, 100, 0, FAKE_S + 4, FAKE_WS, ws)[0] == B.ARL2_ERR_INVALID_ARG
    code, msg = _code(B.arl2_state_init, st, 1, 2, 128, 100, 0, FAKE_S, FAKE_WS, ws - 256)
    assert code == B.ARL2_ERR_INVALID_ARG and "workspace" in msg
    assert _code(B.arl2_state_init, st, 1, 2, 128, 100, 0, FAKE_S, FAKE_WS + 16, ws)[0] == B.ARL2_ERR_INVALID_ARG
    assert _code(B.arl2_state_init, st, 1, 2, 128, 100, 0, FAKE_S, None, ws)[0] == B.ARL2_ERR_INVALID_ARG
    # state overlapping its workspace
    assert _code(B.arl2_state_init, st, 1, 2, 128, 100, 0, FAKE_WS, FAKE_WS, ws)[0] == B.ARL2_ERR_INVALID_ARG
    assert st.magic == 0, "a failed init must leave the descriptor untouched"


def _fake_state(B, Bn=1, H=2, d=128, L=100, dtype=0):
    """A descriptor that passes the state checks, pointing at fake memory."""
    st = B.arl2_state()
    st.B, st.H, st.d, st.L, st.dtype = Bn, H, d, L, dtype
    st.magic = 0x41524C32
    st.S = FAKE_S
    st.ws = FAKE_WS
    st.ws_bytes = B.arl2_workspace_bytes(Bn, H, d, L, dtype)
    return st


Q, K, V, W, OUT, AL, BE = (0x7E0000000000 + i * 0x1000000000 for i in range(7))


def test_frame_forward_validation(B):
    st = _fake_state(B)
    E = B.ARL2_ERR_INVALID_ARG
    assert _code(B.arl2_frame_forward, Q, K, V, W, B.arl2_state(), AL, BE, OUT, 1)[0] == E
    assert _code(B.arl2_frame_forward, Q, K, V, W, st, AL, BE, OUT, 2)[0] == E
    assert _code(B.arl2_frame_forward, Q, K, V, W, st, AL, BE, OUT, -1)[0] == E
    assert _code(B.arl2_frame_forward, None, K, V, W, st, AL, BE, OUT, 0)[0] == E
    assert _code(B.arl2_frame_forward, Q, K, V, None, st, AL, BE, OUT, 0)[0] == E
    assert _code(B.arl2_frame_forward, Q + 2, K, V, W, st, AL, BE, OUT, 0)[0] == E
    assert _code(B.arl2_frame_forward, Q, K, V, W, st, None, BE, OUT, 1)[0] == E
    assert _code(B.arl2_frame_forward, Q, K, V, W, st, AL, None, OUT, 1)[0] == E
    assert _code(B.arl2_frame_forward, Q, K, V, W, st, AL + 2, BE, OUT, 1)[0] == E
    # out aliasing an input, the state or the workspace
    assert "overlaps" in _code(B.arl2_frame_forward, Q, K, V, W, st, AL, BE, Q + 256, 0)[1]
    assert _code(B.arl2_frame_forward, Q, K, V, W, st, AL, BE, FAKE_S, 0)[0] == E
    assert _code(B.arl2_frame_forward, Q, K, V, W, st, AL, BE, FAKE_WS + 1024, 0)[0] == E
    # an input overlapping the state (it would be overwritten by the update)
    assert _code(B.arl2_frame_forward, FAKE_S, K, V, W, st, AL, BE, OUT, 1)[0] == E
    # beta overlapping the state
    assert _code(B.arl2_frame_forward, Q, K, V, W, st, AL, FAKE_S, OUT, 1)[0] == E
    # out overlapping alpha or beta on a clean pass (the update reads both
    # after or while out is written)
    assert "alpha/beta" in _code(B.arl2_frame_forward, Q, K, V, W, st, OUT + 64, BE, OUT, 1)[1]
    assert "alpha/beta" in _code(B.arl2_frame_forward, Q, K, V, W, st, AL, OUT + 512, OUT, 1)[1]
    # a workspace that is too small for the state's shape
    st.ws_bytes -= 256
    assert _code(B.arl2_frame_forward, Q, K, V, W, st, AL, BE, OUT, 0)[0] == E
    st2 = _fake_state(B, d=32)
    assert _code(B.arl2_frame_forward, Q, K, V, W, st2, AL, BE, OUT, 0)[0] == B.ARL2_ERR_UNSUPPORTED
    assert B.arl2_last_error()  # the detail of the last failure is kept


def test_gated_frame_forward_validation(B):
    st = _fake_state(B)
    E = B.ARL2_ERR_INVALID_ARG
    g = B.arl2_frame_forward_gated
    assert "gate" in _code(g, Q, K, V, W, st, AL, 2, BE, OUT, 1)[1]
    assert _code(g, Q, K, V, W, st, AL, -1, BE, OUT, 0)[0] == E
    assert _code(g, Q, K, V, W, st, None, B.ARL2_GATE_ELEMENTWISE, BE, OUT, 1)[0] == E
    # an elementwise alpha ([B][H][d] floats) that reaches into the state
    assert _code(g, Q, K, V, W, st, FAKE_S - 512, B.ARL2_GATE_ELEMENTWISE, BE, OUT, 1)[0] == E
    assert _code(g, Q, K, V, W, st, AL, B.ARL2_GATE_HEADWISE, BE, OUT, 7)[0] == E
    # out overlapping the elementwise alpha or beta on a clean pass
    assert "alpha/beta" in _code(g, Q, K, V, W, st, OUT + 4096, B.ARL2_GATE_ELEMENTWISE, BE,
                                 OUT, 1)[1]
    assert "alpha/beta" in _code(g, Q, K, V, W, st, AL, B.ARL2_GATE_ELEMENTWISE, OUT + 16,
                                 OUT, 1)[1]


def test_noalloc_pass_validation(B):
    """The no-allocation pass validates like arl2_frame_forward and rejects a
    shape whose scratch need exceeds the library's array, before any HIP
    call; a state bound without a workspace is refused by the other passes."""
    E = B.ARL2_ERR_INVALID_ARG
    f = B.arl2_frame_forward_noalloc
    import re as _re
    hdr = open(HEADER).read()
    m = _re.search(r"#define ARL2_NOALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", hdr)
    assert m and int(m.group(1)) << int(m.group(2)) == B.ARL2_NOALLOC_SCRATCH_BYTES
    # the 480p frame step fits; batched 720p does not
    assert B.arl2_workspace_bytes(1, 12, 128, 1560, 0) <= B.ARL2_NOALLOC_SCRATCH_BYTES
    big = _fake_state(B, Bn=4, H=12, L=3600)
    assert B.arl2_workspace_bytes(4, 12, 128, 3600, 0) > B.ARL2_NOALLOC_SCRATCH_BYTES
    code, msg = _code(f, Q, K, V, W, big, AL, BE, OUT, 1)
    assert code == E and "scratch" in msg
    st = _fake_state(B)
    assert _code(f, Q, K, V, W, B.arl2_state(), AL, BE, OUT, 1)[0] == E
    assert _code(f, Q, K, V, W, st, AL, BE, OUT, 3)[0] == E
    # a state without a workspace: only the no-allocation pass accepts it
    st.ws, st.ws_bytes = None, 0
    assert "noalloc" in _code(B.arl2_frame_forward, Q, K, V, W, st, AL, BE, OUT, 0)[1]
    assert "noalloc" in _code(B.arl2_frame_forward_gated, Q, K, V, W, st, AL, 0, BE, OUT, 0)[1]


def test_state_reset_validation(B):
    E = B.ARL2_ERR_INVALID_ARG
    assert _code(B.arl2_state_reset, B.arl2_state(), None)[0] == E
    st = _fake_state(B)
    assert _code(B.arl2_state_reset, st, FAKE_S + 64)[0] == E   # S0 overlaps S
    assert _code(B.arl2_state_reset, st, FAKE_S + (1 << 30) + 2)[0] == E  # misaligned


def test_softmax_attention_validation(B):
    E = B.ARL2_ERR_INVALID_ARG
    nb = B.arl2_softmax_attention_workspace_bytes(1, 12, 128, 1560, 4680, 0)
    assert nb > 0
    assert B.arl2_softmax_attention_workspace_bytes(1, 12, 128, 1560, 0, 0) == 0
    assert _code(B.arl2_softmax_attention, Q, K, V, 1, 12, 128, 1560, 4680, 0, OUT, FAKE_WS, nb - 1)[0] == E
    assert _code(B.arl2_softmax_attention, Q, K, V, 1, 12, 128, 1560, 4680, 0, OUT, None, nb)[0] == E
    assert _code(B.arl2_softmax_attention, Q, K, V, 1, 12, 128, 1560, 4680, 0, Q, FAKE_WS, nb)[0] == E
    assert _code(B.arl2_softmax_attention, Q, K, V, 1, 12, 48, 1560, 4680, 0, OUT, FAKE_WS, nb)[0] == B.ARL2_ERR_UNSUPPORTED


def test_gate_projections_validation(B):
    E = B.ARL2_ERR_INVALID_ARG
    wsb = B.arl2_gate_projections_workspace_bytes
    nb = wsb(1, 1560, 1536, 12, B.ARL2_BF16)
    assert nb > 0 and nb % 256 == 0
    assert wsb(1, 100, 48, 3, B.ARL2_F32) >= 100 * 3 * 4   # one alpha logit per token and head
    for bad in [(0, 1560, 1536, 12, 0), (1, 0, 1536, 12, 0), (1, 1560, 0, 12, 0),
                (1, 1560, 1536, 0, 0), (1, 1560, 1536, 12, 3), (1, 1560, (1 << 16) + 1, 12, 0)]:
        assert wsb(*bad) == 0
    X, WA, WB, A, BT = Q, K, V, AL, BE
    g = B.arl2_gate_projections
    args = [X, WA, WB, 1, 1560, 1536, 12, 0, A, BT, FAKE_WS, nb]
    def call(**kw):
        a = list(args)
        for i, val in kw.items():
            a[int(i[1:])] = val
        return _code(g, *a)
    assert call(a0=None)[0] == E                      # x NULL
    assert call(a1=WA + 8)[0] == E                    # Wa misaligned
    assert call(a8=None)[0] == E                      # alpha NULL
    assert call(a9=BT + 2)[0] == E                    # beta misaligned
    assert "workspace" in call(a11=nb - 1)[1]
    assert call(a10=FAKE_WS + 16)[0] == E             # ws misaligned
    assert call(a8=X + 64)[0] == E                    # alpha inside x
    assert call(a9=A)[0] == E                         # beta overlaps alpha
    assert call(a10=BT)[0] == E                       # workspace overlaps beta
    assert call(a7=9)[0] == E                         # dtype
    assert call(a4=0)[0] == E                         # L


def test_token_level_validation(B):
    E = B.ARL2_ERR_INVALID_ARG
    st = _fake_state(B)
    nb = B.arl2_token_level_workspace_bytes(1, 2, 128, 100, 0)
    assert nb > 0 and nb % 256 == 0
    assert B.arl2_token_level_workspace_bytes(1, 2, 16, 100, 1) == 0   # token-by-token kernel
    assert B.arl2_token_level_workspace_bytes(1, 2, 64, 100, 0) == 0   # unsupported d
    TL = 0x7F2000000000
    f = B.arl2_frame_forward_token_level
    assert _code(f, Q, K, V, W, st, None, BE, OUT, 0, TL, nb)[0] == E      # alpha on every pass
    assert _code(f, Q, K, V, W, st, AL, None, OUT, 1, TL, nb)[0] == E
    assert "workspace" in _code(f, Q, K, V, W, st, AL, BE, OUT, 1, TL, nb - 1)[1]
    assert _code(f, Q, K, V, W, st, AL, BE, OUT, 1, None, nb)[0] == E
    assert _code(f, Q, K, V, W, st, AL, BE, OUT, 1, TL + 16, nb)[0] == E
    assert _code(f, Q, K, V, W, st, AL, BE, OUT, 1, FAKE_WS, nb)[0] == E   # overlaps the state's ws
    assert _code(f, Q, K, V, W, st, AL, BE, OUT, 1, OUT, nb)[0] == E       # overlaps out
    assert _code(f, Q, K, V, W, st, AL, BE, OUT, 2, TL, nb)[0] == E


def test_binding_refuses_to_load_without_the_library(repo_root):
    # Importing the package does not load the library; loading the binding
    # from a path with no library raises ImportError (no silent fallback).
    code = "\n".join([
        "import sys",
        "sys.path.insert(0, %r)" % repo_root,
        "import hybrid_softmax_gated_amd as p",
        "assert 'hybrid_softmax_gated_amd.binding' not in sys.modules",
        "import hybrid_softmax_gated_amd.binding as b",
        "b.LIB_PATH = '/nonexistent/libarl2.so'",
        "try:",
        "    b._load()",
        "except ImportError:",
        "    print('raised')",
    ])
    r = subprocess.run(["python", "-c", code], capture_output=True, text=True)
    assert "raised" in r.stdout, r.stderr


def test_bench_refuses_more_than_one_gpu(repo_root):
    """The benchmark measures one GPU; asking for more exits with status 2
    and says so, before touching any device."""
    r = subprocess.run([sys.executable, os.path.join(repo_root, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "--gpus 2 is not supported" in r.stderr
    assert r.stdout == ""
