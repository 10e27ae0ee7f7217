"""The host side of the C ABI (argument checks, workspace arithmetic, status
strings: mla_api.cpp) under AddressSanitizer and UndefinedBehaviorSanitizer.

A copy of the library whose host code is built with -fsanitize=address and
-fsanitize=undefined (host-only flags; the kernels are the ordinary objects)
runs test_abi_cpu.py in a child interpreter with the ASan runtime preloaded.
Any sanitizer report fails the child (UBSan halts on its first error).
CPU only: nothing here is launched on a GPU.
"""
import os
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


def test_abi_checks_under_asan_and_ubsan():
    if os.environ.get("LD_PRELOAD"):
        pytest.skip("another library is already preloaded into this process tree")
    from mla_latent_kv_15_amd import build
    try:
        runtime = build.asan_runtime()
    except RuntimeError as e:
        pytest.skip(str(e))
    lib_path = build.build_sanitized(verbose=False)
    env = dict(os.environ, MLA_LIBRARY=lib_path, LD_PRELOAD=runtime,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(HERE, "test_abi_cpu.py")],
                       env=env, capture_output=True, text=True, timeout=600,
                       cwd=os.path.dirname(HERE))
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "Sanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert " passed" in out, out[-2000:]
