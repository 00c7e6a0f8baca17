"""Build libpagedattn.so in-tree with hipcc for gfx950.

Every translation unit under csrc/ is compiled to an object file in
parallel (HIP sources for the device and the host, plain C++ sources for the
host only) and linked into ``paged_kv_cache_49_amd/libpagedattn.so``.
Usage: ``python -m paged_kv_cache_49_amd.build`` (or build() from Python).

``--sanitize`` instead builds the host-only parts (the block manager and
the status code, plain C++) with g++ under AddressSanitizer +
UndefinedBehaviorSanitizer and under ThreadSanitizer, as
``_build/sanitize/libpagedattn_host_{asan,tsan}.so``. They export the
block-manager half of the C ABI; load one with ``PA_LIBRARY=<path>`` and the
matching runtime preloaded (``LD_PRELOAD=$(gcc -print-file-name=libasan.so)``).
No device code is built with a sanitizer.
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
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libpagedattn.so")

ARCH = "gfx950"
COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", f"-I{INCLUDE}", f"-I{CSRC}"]
# Packed fp32 ops stay off: the compiler would otherwise fuse fp32 pairs into
# v_pk_* instructions.
HIP_FLAGS = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-munsafe-fp-atomics"]


def _hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libpagedattn)")


def _compile(src: str, hipcc: str, verbose: bool) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    if src.endswith(".hip"):
        cmd = [hipcc, *HIP_FLAGS, *COMMON, "-c", src, "-o", obj]
    else:
        cmd = [hipcc, "-x", "c++", *COMMON, "-c", src, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the packed-fp32 feature and says so; drop that line
    noise = "is not a recognized feature for this target"
    msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"compiling {os.path.basename(src)} failed:\n{msg}")
    if msg.strip() and verbose:
        print(msg, flush=True)
    return obj


def build(verbose: bool = False, jobs: int = 8) -> str:
    """Compile every source and link libpagedattn.so; returns its path."""
    hipcc = _hipcc()
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp")))
    with cf.ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        objs = list(ex.map(lambda s: _compile(s, hipcc, verbose), srcs))
    tmp = LIB + ".tmp"
    cmd = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"linking libpagedattn.so failed:\n{r.stdout}{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


# host-only sources (no HIP), and the flags of each sanitizer build
HOST_SOURCES = ["block_manager.cpp", "status.cpp"]
SANITIZE = {
    "asan": ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"],
    "tsan": ["-fsanitize=thread"],
}


def sanitize_flags(kind: str) -> list:
    """g++ flags of a sanitizer build of host code (``asan``: ASan + UBSan)."""
    return ["-std=c++17", "-O1", "-g", "-pthread", f"-I{INCLUDE}", f"-I{CSRC}", *SANITIZE[kind]]


def build_sanitized(kind: str, verbose: bool = False) -> str:
    """The host-only library (block manager + status) built with g++ under
    ``kind`` (``asan`` or ``tsan``); returns its path."""
    out_dir = os.path.join(BUILD, "sanitize")
    os.makedirs(out_dir, exist_ok=True)
    out = os.path.join(out_dir, f"libpagedattn_host_{kind}.so")
    cmd = ["g++", *sanitize_flags(kind), "-shared", "-fPIC", *[os.path.join(CSRC, f) for f in HOST_SOURCES],
           "-o", out]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"sanitized host build ({kind}) failed:\n{r.stdout}{r.stderr}")
    return out


if __name__ == "__main__":
    if "--sanitize" in sys.argv:
        for k in SANITIZE:
            print(build_sanitized(k, verbose="-v" in sys.argv))
    else:
        print(build(verbose="-v" in sys.argv))
