"""The host layer of the library (argument checks, decoder state, dry-run
schedules) under AddressSanitizer and UndefinedBehaviorSanitizer: the
CPU-only ABI tests run against a host-sanitized build of the same sources,
stopping at the first report.  Builds that library when it is missing or
older than its sources."""

import os
import subprocess
import sys

import pytest

from autoregressive_transformer_decode_amd import build as bld

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

pytestmark = pytest.mark.slow


def _stale() -> bool:
    if not os.path.exists(bld.ASAN_LIB):
        return True
    t = os.path.getmtime(bld.ASAN_LIB)
    srcs = [os.path.join(bld.CSRC, s) for s in bld.SOURCES]
    srcs += [os.path.join(bld.CSRC, "internal.h"), os.path.join(ROOT, "include", "atd.h")]
    return any(os.path.getmtime(p) > t for p in srcs)


def test_abi_cpu_under_asan_and_ubsan():
    if _stale():
        bld.build(sanitize=True)
    rt = bld.sanitizer_runtime()
    env = dict(os.environ)
    env.update(ATD_LIBRARY=bld.ASAN_LIB,
               LD_PRELOAD=os.path.join(rt, "libclang_rt.asan-x86_64.so"),
               LD_LIBRARY_PATH=rt + os.pathsep + env.get("LD_LIBRARY_PATH", ""),
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi_cpu.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    assert r.returncode == 0, r.stdout[-4000:] + r.stderr[-4000:]
    assert "passed" in r.stdout and "AddressSanitizer" not in r.stderr, r.stderr[-2000:]
