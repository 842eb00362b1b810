"""Build libgqa.so (the gfx950 HIP kernels and the C ABI) in-tree with hipcc.

    python -m grouped_query_attention_gemv_amd.build [--verbose]

Objects go to ``_build/`` at the repository root; the shared library is
written next to this file, where the Python binding loads it.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libgqa.so")
ARCH = "gfx950"

SOURCES = ["api.hip", "rope.hip", "decode.hip", "prefill.hip", "norm.hip", "vocab.hip"]

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-function",
    "-Wno-unused-variable",
    # keep the compiler from forming packed fp32 arithmetic
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{INCLUDE}",
    f"-I{CSRC}",
]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; ROCm is required to build libgqa.so")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out, flush=True)


# Host-side AddressSanitizer + UndefinedBehaviorSanitizer build of the same
# sources (argument validation, workspace carving, dispatch).  Every
# sanitizer flag applies to the host compilation only; the gfx950 code is
# built as usual.  Load it with the clang ASan runtime preloaded, e.g.
#   LD_PRELOAD=<libclang_rt.asan-x86_64.so> GQA_LIB=_build/asan/libgqa.so python ...
SANITIZE_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                  "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=all",
                  "-Xarch_host", "-shared-libsan"]
ASAN_LIB = os.path.join(BUILD, "asan", "libgqa.so")


def asan_runtime() -> str:
    """Path of the clang AddressSanitizer runtime that hipcc links against."""
    r = subprocess.run([_hipcc(), "-print-file-name=libclang_rt.asan-x86_64.so"],
                       capture_output=True, text=True)
    return r.stdout.strip()


def build(verbose: bool = False, sanitize: bool = False) -> str:
    """Compile every source for gfx950 and link libgqa.so; returns its path.
    With sanitize, the host side is instrumented and the library goes to
    _build/asan/ instead (for the host tests only)."""
    hipcc = _hipcc()
    out_dir = os.path.join(BUILD, "asan") if sanitize else BUILD
    lib = ASAN_LIB if sanitize else LIB
    extra = SANITIZE_FLAGS if sanitize else []
    os.makedirs(out_dir, exist_ok=True)
    objs = []
    jobs = []
    for src in SOURCES:
        obj = os.path.join(out_dir, src.replace(".hip", ".o"))
        objs.append(obj)
        jobs.append([hipcc, *HIPCC_FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj])
    with ThreadPoolExecutor(max_workers=min(len(jobs), 8)) as ex:
        list(ex.map(lambda c: _run(c, verbose), jobs))
    tmp = lib + ".tmp"
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *extra, *objs, "-o", tmp], verbose)
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    path = build(verbose="--verbose" in sys.argv, sanitize="--sanitize" in sys.argv)
    print(path)
