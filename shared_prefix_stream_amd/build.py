"""Build libppattn.so in-tree with hipcc for gfx950.

    python -m shared_prefix_stream_amd.build        # or: python shared_prefix_stream_amd/build.py

Every translation unit under csrc/ is compiled to an object in parallel, then
linked into shared_prefix_stream_amd/libppattn.so.  Flags: gfx950 only, -O3,
and packed-FP32 instructions disabled in the device code (the compiler would
otherwise form v_pk_{add,mul,fma}_f32 from plain float code).

build_host_asan(path) makes a second library whose host code (the argument
validation, planning and launch code) is built with AddressSanitizer; the
device code is the same.  A process that loads it needs the matching ASan
runtime (asan_runtime()) loaded first.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libppattn.so")
BUILD_DIR = os.path.join(PKG, "_build")
ARCH = "gfx950"

DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall", "-Wno-unused-function",
          "-I", os.path.join(ROOT, "include"), "-I", CSRC]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libppattn)")


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _compile(hipcc: str, src: str, extra, build_dir: str = BUILD_DIR):
    obj = os.path.join(build_dir, os.path.basename(src) + ".o")
    cmd = [hipcc, *COMMON, *DEVICE_FLAGS, *extra, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the packed-fp32 feature and says so; harmless
    noise = "'-packed-fp32-ops' is not a recognized feature"
    err = "\n".join(line for line in r.stderr.splitlines() if noise not in line)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{err}")
    return obj, err


def _build_to(lib: str, build_dir: str, extra=(), link_extra=(), verbose: bool = False) -> str:
    hipcc = _hipcc()
    os.makedirs(build_dir, exist_ok=True)
    srcs = sources()
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        results = list(ex.map(lambda s: _compile(hipcc, s, list(extra), build_dir), srcs))
    for _, err in results:
        if err.strip() and verbose:
            print(err, file=sys.stderr)
    tmp = lib + ".tmp"
    cmd = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *link_extra, "-o", tmp, *[o for o, _ in results]]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stderr}")
    os.replace(tmp, lib)
    return lib


def build(verbose: bool = False, extra=()) -> str:
    return _build_to(LIB, BUILD_DIR, extra, verbose=verbose)


# host pass only (-Xarch_host): the device code is built as in build()
ASAN_HOST_FLAGS = ["-Xarch_host", "-O1", "-Xarch_host", "-g", "-Xarch_host", "-fsanitize=address",
                   "-Xarch_host", "-fno-omit-frame-pointer"]


def build_host_asan(lib: str, build_dir: str) -> str:
    """libppattn with AddressSanitizer on its host code, written to `lib`."""
    return _build_to(lib, build_dir, ASAN_HOST_FLAGS, ["-Xarch_host", "-fsanitize=address", "-shared-libasan"])


def asan_runtime() -> str:
    """Path of the compiler's shared ASan runtime (to be loaded before a
    library built by build_host_asan)."""
    clang = os.path.join(os.path.dirname(os.path.realpath(_hipcc())), "..", "llvm", "bin", "clang")
    for cand in (clang, "/opt/rocm/llvm/bin/clang"):
        if os.path.exists(cand):
            r = subprocess.run([cand, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
            path = r.stdout.strip()
            if r.returncode == 0 and os.path.isabs(path) and os.path.exists(path):
                return path
    raise RuntimeError("the compiler's shared ASan runtime was not found")


if __name__ == "__main__":
    print(build(verbose=True))
