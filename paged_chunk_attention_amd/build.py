"""Build liboomb.so (the HIP library behind include/oomb.h) in-tree for gfx950.

    python -m paged_chunk_attention_amd.build        # or: build() from Python

Every source is compiled with hipcc for gfx950 only; objects go to _build/ at the
repository root and the shared library next to this file, where the binding loads it.
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
BUILD_DIR = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "liboomb.so")
ARCH = "gfx950"

SOURCES = {
    # the mean-key summary's float arithmetic is fixed too (no fused multiply-adds)
    "paging.hip": ["-ffp-contract=off"],
    # the selector's float arithmetic must not be contracted into fused multiply-adds
    "select.hip": ["-ffp-contract=off"],
    "attn_scalar.hip": [],
    # no NaN ever reaches the softmax maxima (masking uses -inf): lets fmaxf skip the
    # NaN-quieting v_max of each operand
    "attn_fwd_mfma.hip": ["-fno-honor-nans"],
    # the ILP-first scheduler measures 2-3% faster for the dQ pass
    "attn_dq_mfma.hip": ["-mllvm", "-amdgpu-sched-strategy=max-ilp"],
    "attn_dkdv_mfma.hip": [],
    "offload.hip": [],
    # fp32 rotation, fp64 angles: no contraction, so the rounding is the plain one
    "rope.hip": ["-ffp-contract=off"],
    "api.cpp": [],
    "profiling.cpp": [],
}

COMMON = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # packed fp32 VALU instructions are kept out of every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
    "-Wall", "-Wno-unused-function", "-Wno-unused-command-line-argument",
]


# Sources of the matrix-core attention kernels, whose hash tags measured profiles: the
# kernels, the headers they include, and launch.hpp, which also holds the host rules that
# decide how the passes split their work.
MFMA_SOURCES = ["device_common.hpp", "launch.hpp", "mfma_tiles.hpp", "attn_fwd_mfma.hip",
                "attn_dq_mfma.hip", "attn_dkdv_mfma.hip"]


def mfma_source_hash() -> str:
    """First 16 hex digits of the sha256 over the matrix-core kernel sources and their
    compile flags (a profile taken from other sources no longer describes the kernels)."""
    import hashlib
    h = hashlib.sha256()
    for name in MFMA_SOURCES:
        h.update(name.encode())
        h.update(open(os.path.join(CSRC, name), "rb").read())
        h.update(" ".join(SOURCES.get(name, [])).encode())
    return h.hexdigest()[:16]


def hipcc() -> str:
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        raise RuntimeError("hipcc not found: a ROCm toolchain is required to build liboomb.so")
    return exe


def _compile(src: str, extra, verbose: bool) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    lang = ["-x", "hip"] if src.endswith(".cpp") else []
    cmd = [hipcc(), *lang, *COMMON, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{res.stdout}\n{res.stderr}")
    warn = "\n".join(l for l in res.stderr.splitlines()
                     if "packed-fp32-ops" not in l and l.strip())
    if warn and verbose:
        print(warn, file=sys.stderr)
    return obj


def build(verbose: bool = False) -> str:
    """Compile every source and link liboomb.so; returns the library path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 4)) as ex:
        objs = list(ex.map(lambda kv: _compile(kv[0], kv[1], verbose), SOURCES.items()))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "-shared", f"--offload-arch={ARCH}", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
