"""The host ABI tests once more against the library's host code built with
AddressSanitizer and UndefinedBehaviorSanitizer (the device code is built
uninstrumented; no GPU is used): every argument check, workspace size query
and early return runs instrumented, in a subprocess with the shared
sanitizer runtime preloaded, and any report fails the run."""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _stale(target, sources):
    if not os.path.exists(target):
        return True
    t = os.path.getmtime(target)
    return any(os.path.getmtime(s) > t for s in sources)


def test_host_abi_under_asan_and_ubsan():
    from token_tree_attention_amd import build as B
    if not os.path.exists(B.HIPCC) or not os.path.exists(B.CLANGXX):
        pytest.skip("hipcc / clang++ not available")
    sources = [os.path.join(B.CSRC, s) for s in B.SOURCES] + [os.path.join(ROOT, "include", "treeverify.h"),
                                                             os.path.join(B.CSRC, "ttv_device.h")]
    lib = B.build_host_sanitized() if _stale(B.SANITIZED, sources) else B.SANITIZED
    env = dict(os.environ)
    env.update(LD_PRELOAD=B.sanitizer_runtime(), TTV_LIBRARY=lib,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi_host.py")], cwd=ROOT, env=env,
                       stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, timeout=600)
    assert r.returncode == 0, r.stdout[-4000:]
    assert "ERROR: AddressSanitizer" not in r.stdout and "runtime error" not in r.stdout, r.stdout[-4000:]
