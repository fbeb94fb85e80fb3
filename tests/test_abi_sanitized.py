"""The C-ABI argument checks (tests/test_abi.py) run again against libsala_asan.so, whose host
code is built with AddressSanitizer and UndefinedBehaviorSanitizer (hybrid_sparse_linear_causal_amd
/build.py, build_asan): every validation path of the entry points runs instrumented, on the CPU,
with the clang ASan runtime preloaded into a child interpreter. Any sanitizer report fails."""

import os
import subprocess
import sys

import pytest

from conftest import ROOT

ASAN_LIB = os.path.join(ROOT, "hybrid_sparse_linear_causal_amd", "libsala_asan.so")


@pytest.mark.skipif(not os.path.exists(ASAN_LIB), reason="libsala_asan.so not built")
def test_abi_checks_under_asan_and_ubsan():
    from hybrid_sparse_linear_causal_amd.build import asan_runtime

    rt = asan_runtime()
    if rt is None:
        pytest.skip("clang ASan runtime not found")
    env = dict(os.environ, LD_PRELOAD=rt, SALA_LIBRARY=ASAN_LIB,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi.py")], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=600)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in r.stdout, out[-2000:]
