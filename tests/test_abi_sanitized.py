"""The CPU ABI checks of tests/test_abi.py, run against a build whose host
code carries AddressSanitizer and UndefinedBehaviorSanitizer
(diffusion_transformer_dit_amd/build_sanitized.py): the argument checks,
workspace arithmetic and stack bookkeeping must not read or write out of
bounds or hit undefined behaviour on any of the tested paths.  Runs on the
CPU only; the clang ASan runtime is preloaded into a child interpreter."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_abi_checks_under_host_sanitizers():
    from diffusion_transformer_dit_amd import build_sanitized as BS
    rt = BS.asan_runtime()
    if not rt:
        pytest.skip("clang ASan runtime not found under /opt/rocm/llvm")
    lib = BS.build()
    env = dict(os.environ, DIT_LIB=lib, LD_PRELOAD=rt, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_abi.py"), "-q",
                        "-p", "no:cacheprovider"], cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert " passed" in r.stdout
