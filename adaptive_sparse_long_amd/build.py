"""Build libdash.so (gfx950) in-tree with hipcc.

    python -m adaptive_sparse_long_amd.build        # or build() from Python

Every HIP source is compiled for gfx950 only, with packed-FP32 instruction
selection turned off (-Xclang -target-feature -Xclang -packed-fp32-ops), into
objects under _build/, then linked into adaptive_sparse_long_amd/libdash.so.
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
BUILD_DIR = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libdash.so")

SOURCES = [
    "api.cpp",
    "summarize.hip",
    "route.hip",
    "sparse_prefill.hip",
    "sparse_decode.hip",
    "entmax_attn.hip",
    "entmax_attn_bwd.hip",
    "dash_bwd.hip",
    "entmax_rows.hip",
]

ARCH = "gfx950"


def _hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the library needs ROCm's hipcc to build")


def _flags():
    return [
        f"--offload-arch={ARCH}",
        "-O3",
        "-std=c++17",
        "-fPIC",
        "-Wall",
        "-Wno-unused-function",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", INCLUDE,
        "-I", CSRC,
    ]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass warns that it does not know the packed-fp32 feature: harmless
    err = "\n".join(l for l in res.stderr.splitlines() if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"command failed ({res.returncode}): {' '.join(cmd)}\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)


def _stale(obj: str, src: str) -> bool:
    """True if obj is missing or older than its source or any shared header."""
    if not os.path.exists(obj):
        return True
    deps = [src] + [os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hpp")]
    deps.append(os.path.join(INCLUDE, "dash.h"))
    t = os.path.getmtime(obj)
    return any(os.path.getmtime(p) > t for p in deps)


def build(verbose: bool = False, jobs: int | None = None, only_changed: bool = False) -> str:
    """Compile every source (only_changed: only those newer than their object)
    and link libdash.so; returns the library path."""
    hipcc = _hipcc()
    os.makedirs(BUILD_DIR, exist_ok=True)
    objs = []
    cmds = []
    for src in SOURCES:
        obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
        objs.append(obj)
        if only_changed and not _stale(obj, os.path.join(CSRC, src)):
            continue
        lang = ["-x", "hip"] if src.endswith(".cpp") else []
        cmds.append([hipcc, *_flags(), *lang, "-c", os.path.join(CSRC, src), "-o", obj])
    jobs = jobs or max(1, min(len(cmds), os.cpu_count() or 2))
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        list(ex.map(lambda c: _run(c, verbose), cmds))
    tmp = LIB + ".tmp"
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs], verbose)
    os.replace(tmp, LIB)
    return LIB


# Host-code checking build: the C ABI layer (api.cpp: argument validation,
# workspace layouts, launch set-up) compiled with AddressSanitizer and
# UndefinedBehaviorSanitizer on its host side only (GPU code is never
# instrumented), linked with the regular kernel objects. Loaded by the CPU ABI
# tests with the ASan runtime preloaded; never by the product path.
SAN_LIB = os.path.join(BUILD_DIR, "libdash_hostsan.so")
SAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=undefined"]


def build_host_sanitized(verbose: bool = False) -> str:
    """Build _build/libdash_hostsan.so (needs the regular objects: run build() first)."""
    hipcc = _hipcc()
    objs = []
    for src in SOURCES:
        obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
        if not os.path.exists(obj):
            raise RuntimeError(f"{obj} is missing: build the library first")
        objs.append(obj)
    api_obj = os.path.join(BUILD_DIR, "api_hostsan.o")
    _run([hipcc, *_flags(), *SAN_FLAGS, "-O1", "-x", "hip", "-c", os.path.join(CSRC, "api.cpp"), "-o", api_obj], verbose)
    objs = [api_obj if o.endswith(os.sep + "api.o") else o for o in objs]
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-shared-libsan", *SAN_FLAGS, "-o", SAN_LIB, *objs],
         verbose)
    return SAN_LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, only_changed="--changed" in sys.argv))
    if "--host-sanitize" in sys.argv:
        print(build_host_sanitized(verbose="-v" in sys.argv))
