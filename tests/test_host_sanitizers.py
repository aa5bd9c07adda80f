"""The host side of the C ABI under AddressSanitizer and UndefinedBehaviorSanitizer.

Builds the library once more with the sanitizers on its host code only (each
flag behind -Xarch_host; the gfx950 device code is built as usual), then runs
the CPU tests that drive the host code (argument checks of every entry point,
the block pool) in a child process with the sanitizer runtime preloaded.  Any
report aborts the child, so the test passes only if both suites run clean.
No GPU is used: with no device the entry points stop at their checks or at the
first HIP call.
"""
import glob
import os
import shutil
import subprocess
import sys

import pytest

from mla_latent_kv_02_amd import build as mla_build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HOST_FLAGS = ["-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=undefined",
              "-g", "-fno-omit-frame-pointer"]


def _asan_runtime():
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


@pytest.mark.timeout(900)
def test_abi_and_block_pool_are_clean_under_asan_and_ubsan(tmp_path):
    runtime = _asan_runtime()
    if runtime is None or shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"):
        pytest.skip("no hipcc or no clang sanitizer runtime")
    lib = str(tmp_path / "libmla_sanitized.so")
    mla_build.build(lib_path=lib, host_flags=HOST_FLAGS, synth=False, jobs=8)
    env = dict(os.environ)
    env.update(LD_PRELOAD=runtime, MLA_LIBRARY=lib,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    # -s: a report goes to the child's stderr before the abort, not into
    # pytest's capture buffer
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-s", "-p", "no:cacheprovider",
                        "tests/test_abi.py", "tests/test_block_pool.py"],
                       cwd=ROOT, env=env, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True,
                       timeout=600)
    reports = [l for l in r.stdout.splitlines()
               if "runtime error:" in l or "AddressSanitizer" in l or "UndefinedBehaviorSanitizer" in l]
    assert r.returncode == 0 and not reports, r.stdout[-4000:]
    assert " passed" in r.stdout.splitlines()[-1]
