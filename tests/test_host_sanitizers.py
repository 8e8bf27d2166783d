"""The C ABI's host code (argument validation, workspace arithmetic, the host helpers)
under AddressSanitizer and UndefinedBehaviorSanitizer.

The library is rebuilt with the host side instrumented (device code unchanged; no GPU is
used) and ``test_boundary.py`` runs against it in a subprocess with the ASan runtime
preloaded.  Any sanitizer report aborts that run: UBSan is built without recovery, so a
signed overflow in the size checks (they are fed sizes up to INT64_MAX) fails the test.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _asan_runtime():
    clang = "/opt/rocm/lib/llvm/bin/clang"
    if not os.path.exists(clang):
        return None
    out = subprocess.run([clang, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True,
                         text=True).stdout.strip()
    return out if out and os.path.isabs(out) and os.path.exists(out) else None


@pytest.mark.skipif(os.environ.get("VP_LMHEAD_LIB") is not None, reason="already the sanitized run")
def test_boundary_under_asan_and_ubsan():
    rt = _asan_runtime()
    if rt is None or shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"):
        pytest.skip("hipcc or the clang ASan runtime is not available")
    sys.path.insert(0, os.path.join(ROOT, "vocab_lm_head_amd"))
    import importlib.util
    spec = importlib.util.spec_from_file_location(
        "vp_build", os.path.join(ROOT, "vocab_lm_head_amd", "build.py"))
    build = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(build)
    lib = build.build(verbose=False, sanitize=True)
    env = dict(os.environ, VP_LMHEAD_LIB=lib, LD_PRELOAD=rt,
               ASAN_OPTIONS="detect_leaks=0:verify_asan_link_order=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_boundary.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    tail = (r.stdout + r.stderr)[-4000:]
    assert r.returncode == 0, f"sanitized boundary run failed:\n{tail}"
    assert "passed" in r.stdout and "ERROR: AddressSanitizer" not in tail and "runtime error" not in tail
