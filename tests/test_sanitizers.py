"""Host sanitizers (AddressSanitizer + UndefinedBehaviorSanitizer) over the
C ABI's validation paths and the oracle.  The ABI library's host code and
the oracle are rebuilt with the sanitizers, and the argument-error tests of
the ABI and the oracle's pin tests run again in a child process that loads
those builds under clang's ASan runtime; any sanitizer report fails the
test.  CPU only: the ABI tests make no HIP call that reaches a device."""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _asan_runtime():
    libs = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return libs[-1] if libs else None


def test_abi_and_oracle_under_asan_ubsan():
    rt = _asan_runtime()
    if rt is None:
        pytest.skip("clang's ASan runtime is not installed")
    sys.path.insert(0, ROOT)
    from block_scaled_fp4_03_amd import build as b
    import oracle
    lib = b.build_sanitized()
    oracle.build_sanitized()
    env = dict(os.environ, LD_PRELOAD=rt, FP4_LIB_PATH=lib, ORACLE_SANITIZE="1",
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    cmd = [sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu",
           "tests/test_abi.py", "tests/test_oracle_pins.py", "tests/test_codecs.py", "tests/test_oracle_mxfp8.py",
           "tests/test_output_checkers.py", "-k", "not wrappers and not sanitizers"]
    r = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in out
