"""Build libkvq.so in-tree with hipcc for gfx950.

    python -m quantized_paged_kv_absmax_amd.build [--host-sanitizers]

Objects go to quantized_paged_kv_absmax_amd/_build/, the shared library to
quantized_paged_kv_absmax_amd/lib/libkvq.so, and bench.py's page-read probe to
lib/libkvq_probe.so (with --host-sanitizers,
lib/libkvq_hostsan.so: the C ABI's host code under ASan and UBSan).  Every call
rebuilds.
"""

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIBDIR = os.path.join(PKG, "lib")
LIB = os.path.join(LIBDIR, "libkvq.so")
# a measurement aid for bench.py (a read of the decode's pages, no compute), not
# part of libkvq.so's C ABI
PROBE_LIB = os.path.join(LIBDIR, "libkvq_probe.so")
PROBE_SOURCE = "read_probe.hip"

ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CFLAGS = [
    "-O3", "-fPIC", "-std=c++17", f"--offload-arch={ARCH}",
    # packed fp32 instructions are kept out of every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA accumulators in VGPRs: the softmax rescale and the integer-logit
    # combine then touch them without AGPR <-> VGPR copies
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-Wall", "-Wno-unused-function",
    f"-I{os.path.join(ROOT, 'include')}",
]
SOURCES = ["kvq_api.cpp", "calibrate.hip", "cache_write.hip", "decode.hip", "verify.hip"]


def _compile(src):
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    lang = ["-x", "hip"]
    cmd = [HIPCC, *CFLAGS, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj, r.stderr


def build(verbose=False):
    os.makedirs(BUILD, exist_ok=True)
    os.makedirs(LIBDIR, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(8, len(SOURCES) + 1)) as ex:
        results = list(ex.map(_compile, SOURCES + [PROBE_SOURCE]))
    probe_obj = results.pop()[0]
    objs = [o for o, _ in results]
    if verbose:
        for (o, err) in results:
            warn = "\n".join(l for l in err.splitlines() if "packed-fp32-ops" not in l and l.strip())
            if warn:
                print(warn, file=sys.stderr)
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    tmp = PROBE_LIB + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", probe_obj, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, PROBE_LIB)
    return LIB


# Host sanitizer build: kvq_api.cpp (every argument check and the launch
# geometry) with AddressSanitizer and UndefinedBehaviorSanitizer on its host
# code only, linked with the ordinary device objects into lib/libkvq_hostsan.so.
# Load it with the clang ASan runtime preloaded (host_sanitizer_runtime()) and
# KVQ_LIBRARY pointing at it.
HOSTSAN_LIB = os.path.join(LIBDIR, "libkvq_hostsan.so")
HOSTSAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer", "-g"]


def host_sanitizer_runtime():
    """Path of the clang AddressSanitizer runtime that the sanitizer build needs preloaded."""
    root = os.path.join(os.path.dirname(os.path.dirname(HIPCC)), "llvm", "lib", "clang")
    for ver in sorted(os.listdir(root), reverse=True) if os.path.isdir(root) else []:
        cand = os.path.join(root, ver, "lib", "linux", "libclang_rt.asan-x86_64.so")
        if os.path.exists(cand):
            return cand
    raise FileNotFoundError("clang AddressSanitizer runtime not found under " + root)


def build_host_sanitized():
    os.makedirs(BUILD, exist_ok=True)
    os.makedirs(LIBDIR, exist_ok=True)
    others = [s for s in SOURCES if s != "kvq_api.cpp"]
    with ThreadPoolExecutor(max_workers=min(8, len(others))) as ex:
        objs = [o for o, _ in ex.map(_compile, others)]
    san_obj = os.path.join(BUILD, "kvq_api_hostsan.o")
    cmd = [HIPCC, *CFLAGS, *HOSTSAN_FLAGS, "-x", "hip", "-c", os.path.join(CSRC, "kvq_api.cpp"), "-o", san_obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for the host sanitizer build:\n{' '.join(cmd)}\n{r.stderr}")
    tmp = HOSTSAN_LIB + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", san_obj, *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stderr}")
    os.replace(tmp, HOSTSAN_LIB)
    return HOSTSAN_LIB


def clean():
    shutil.rmtree(BUILD, ignore_errors=True)


if __name__ == "__main__":
    if "--host-sanitizers" in sys.argv:
        print(build_host_sanitized())
    else:
        print(build(verbose=True))
