"""The C ABI's host code under AddressSanitizer, on the CPU.

Every source is compiled again with the sanitizer on the host side only
(device code is built as usual), linked into a separate copy of the library,
and the CPU ABI tests (argument validation, symbol exports, profiling
bookkeeping) run against that copy in a child process with the sanitizer
runtime preloaded. A heap or stack overflow, a use after free or a double
free in the validation code fails the test with the sanitizer's report.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

from hybrid_softmax_gated_amd import build as libbuild  # noqa: E402

OUT_DIR = os.path.join(ROOT, "_build", "asan")
LIB = os.path.join(OUT_DIR, "libarl2_asan.so")


def _asan_runtime(cc):
    r = subprocess.run([cc, "-print-file-name=libclang_rt.asan-x86_64.so"],
                       capture_output=True, text=True)
    path = r.stdout.strip()
    return path if r.returncode == 0 and os.path.isfile(path) else None


def _build_asan(cc):
    os.makedirs(OUT_DIR, exist_ok=True)
    objs = []
    for src in libbuild.sources():
        obj = os.path.join(OUT_DIR, os.path.basename(src)[:-4] + ".o")
        cmd = [cc, *libbuild.COMMON, "-O1", "-g", "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer", "-c", src, "-o", obj]
        rc, out = libbuild._run(cmd)
        assert rc == 0, out
        objs.append(obj)
    # The sanitizer's symbols stay undefined in the shared object; the
    # preloaded runtime provides them.
    rc, out = libbuild._run([cc, f"--offload-arch={libbuild.ARCH}", "-shared", "-fPIC", *objs,
                             "-o", LIB])
    assert rc == 0, out


def test_abi_validation_under_address_sanitizer():
    try:
        cc = libbuild.hipcc()
    except RuntimeError:
        pytest.skip("hipcc is not available")
    rt = _asan_runtime(cc)
    if rt is None:
        pytest.skip("the compiler has no AddressSanitizer runtime")
    _build_asan(cc)
    env = dict(os.environ)
    env.update({"LD_PRELOAD": rt, "ARL2_LIBRARY": LIB,
                "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=0:halt_on_error=1"})
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi_cpu.py"),
                        "-k", "not bench_refuses and not binding_refuses"],
                       capture_output=True, text=True, env=env, cwd=ROOT, timeout=600)
    report = r.stdout + r.stderr
    assert "AddressSanitizer" not in report, report[-4000:]
    assert r.returncode == 0, report[-4000:]
    assert " passed" in r.stdout
