"""CPU: the C-ABI layer's host code (argument checks, size arithmetic,
error text) under AddressSanitizer and UndefinedBehaviorSanitizer. The
boundary tests run in a child process against libmoe_san.so (api.cpp built
with host-side -fsanitize=address,undefined, undefined behaviour fatal),
with the shared ASan runtime preloaded; any report fails the run."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
                    reason="needs hipcc to build the sanitizer library")
def test_boundary_tests_pass_under_asan_and_ubsan():
    sys.path.insert(0, ROOT)
    from mixture_experts_layer_49_amd import build as b

    lib = b.build_sanitized()
    rt = b.asan_runtime()
    assert os.path.exists(rt), rt
    env = dict(os.environ, MOE_LIB=lib, LD_PRELOAD=rt,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_boundary.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "ERROR: AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert " passed" in out
