"""The C ABI's host code (argument checks, work split, workspace layout in
kvq_api.cpp) built with AddressSanitizer and UndefinedBehaviorSanitizer on the
host side only (lib/libkvq_hostsan.so), and the no-GPU ABI tests run against it
with the clang ASan runtime preloaded: the run must pass with no sanitizer
report.  No GPU is used."""

import os
import shutil
import subprocess
import sys

import pytest

from quantized_paged_kv_absmax_amd import build as kbuild

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

pytestmark = pytest.mark.skipif(shutil.which(kbuild.HIPCC) is None and not os.path.exists(kbuild.HIPCC),
                                reason="hipcc not available")


def _stale():
    if not os.path.exists(kbuild.HOSTSAN_LIB):
        return True
    t = os.path.getmtime(kbuild.HOSTSAN_LIB)
    srcs = [os.path.join(kbuild.CSRC, f) for f in os.listdir(kbuild.CSRC)] + [os.path.join(ROOT, "include", "kvq.h")]
    return any(os.path.getmtime(p) > t for p in srcs)


@pytest.mark.timeout(900)
def test_abi_checks_are_clean_under_host_sanitizers():
    if _stale():
        kbuild.build_host_sanitized()
    syms = subprocess.run(["nm", "-D", kbuild.HOSTSAN_LIB], capture_output=True, text=True).stdout
    assert "__asan_report" in syms and "__ubsan_handle" in syms          # the host code is instrumented
    env = dict(os.environ, KVQ_LIBRARY=kbuild.HOSTSAN_LIB, LD_PRELOAD=kbuild.host_sanitizer_runtime(),
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1", UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi_cpu.py")], capture_output=True, text=True, env=env,
                       cwd=ROOT, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-3000:]
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-3000:]
    assert " passed" in out
