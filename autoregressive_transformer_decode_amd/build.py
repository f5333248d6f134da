"""Build the HIP library in-tree: hipcc for gfx950 -> libatd.so.

    python -m autoregressive_transformer_decode_amd.build [--sanitize]

--sanitize builds libatd_asan.so instead: the same sources with the host code
(argument checks, decoder state, launch sequences) under AddressSanitizer and
UndefinedBehaviorSanitizer; device code is built as usual.  Load it with
ATD_LIBRARY=<path> and the sanitizer runtime preloaded (tests/
test_host_sanitizers.py does this for the CPU-only ABI tests)."""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libatd.so")
SOURCES = ["abi.cpp", "kernels.hip"]
ARCH = "gfx950"

# Packed-FP32 instructions are switched off for all device code.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
# sanitizers on the host side only (each flag behind -Xarch_host)
SANITIZE_FLAGS = ("-Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined "
                  "-Xarch_host -fno-omit-frame-pointer -Xarch_host -fno-sanitize-recover=all").split()
ASAN_LIB = os.path.join(HERE, "libatd_asan.so")


def sanitizer_runtime() -> str:
    """Directory of the compiler's sanitizer runtime (to preload it)."""
    root = os.path.join(os.path.dirname(os.path.realpath(hipcc())), "..", "llvm", "lib", "clang")
    for ver in sorted(os.listdir(root), reverse=True):
        d = os.path.join(root, ver, "lib", "linux")
        if os.path.exists(os.path.join(d, "libclang_rt.asan-x86_64.so")):
            return os.path.realpath(d)
    raise RuntimeError("sanitizer runtime not found under " + root)


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the library)")


def build(verbose: bool = False, sanitize: bool = False) -> str:
    objs = []
    tmp = os.path.join(HERE, "_build_asan" if sanitize else "_build")
    os.makedirs(tmp, exist_ok=True)
    opt = ["-O1", "-g", *SANITIZE_FLAGS] if sanitize else ["-O3"]
    for src in SOURCES:
        obj = os.path.join(tmp, src + ".o")
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        cmd = [hipcc(), *lang, f"--offload-arch={ARCH}", *opt, "-std=c++17", "-fPIC",
               "-Wall", "-Wno-unused-result", *DEVICE_FLAGS,
               "-I", os.path.join(HERE, "..", "include"), "-c",
               os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        objs.append(obj)
    lib = ASAN_LIB if sanitize else LIB
    out_tmp = lib + ".tmp"
    link = ["-shared-libsan", *SANITIZE_FLAGS] if sanitize else []
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *link, "-o", out_tmp, *objs,
           "-ldl"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(out_tmp, lib)
    return lib


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, sanitize="--sanitize" in sys.argv))
