"""The host runtime (argument checks, cache objects, the block allocator,
metadata validation, workspace sizing) under AddressSanitizer and
UndefinedBehaviorSanitizer: the library is rebuilt with both sanitizers on its
host code only (paged_kv_gqa_05_amd/build.py --host-sanitized), and the CPU
ABI tests run against that build in a child process with the sanitizer
runtime preloaded.  Any sanitizer report fails the test.  No kernel runs."""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

pytestmark = pytest.mark.slow


def _asan_runtime():
    libs = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return libs[-1] if libs else None


@pytest.mark.skipif(_asan_runtime() is None, reason="no clang AddressSanitizer runtime in this image")
def test_abi_cpu_tests_under_asan_and_ubsan():
    build = subprocess.run([sys.executable, os.path.join(ROOT, "paged_kv_gqa_05_amd", "build.py"),
                            "--host-sanitized"], capture_output=True, text=True, timeout=900)
    assert build.returncode == 0, build.stdout + build.stderr
    lib = build.stdout.strip().splitlines()[-1]
    env = dict(os.environ, LD_PRELOAD=_asan_runtime(), PKV_LIB_PATH=lib,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    run = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                          os.path.join(ROOT, "tests", "test_abi_cpu.py")],
                         capture_output=True, text=True, timeout=600, env=env, cwd=ROOT)
    out = run.stdout + run.stderr
    assert run.returncode == 0, out[-4000:]
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert " passed" in out
