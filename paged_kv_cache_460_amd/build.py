"""Build libpa.so in-tree with hipcc for gfx950.

    python -m paged_kv_cache_460_amd.build [-v]

Objects go to ``paged_kv_cache_460_amd/_build/``; the shared library to
``paged_kv_cache_460_amd/libpa.so`` (replaced atomically).
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(HERE, "_build")
LIB_PATH = os.path.join(HERE, "libpa.so")

SOURCES = [
    "pa_api.cpp",
    "block_manager.cpp",
    "slots.hip",
    "scatter.hip",
    "plan.hip",
    "decode_bf16.hip",
    "reduce.hip",
    "prefill_bf16.hip",
    "attn_f32.hip",
    "debug_checks.hip",
    "noalloc.hip",
]

ARCH = "gfx950"
# Packed-fp32 VALU forms stay disabled: the compiler must not emit them.
COMMON_FLAGS = [
    "-O3",
    f"--offload-arch={ARCH}",
    "-fPIC",
    "-std=c++17",
    "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE,
    "-I", CSRC,
]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libpa)")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(line for line in res.stderr.splitlines() if noise not in line)
    if res.returncode != 0:
        raise RuntimeError(f"command failed ({res.returncode}): {' '.join(cmd)}\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)


def build(verbose: bool = False, jobs: int = 8) -> str:
    """Compile every source and link libpa.so; returns its path."""
    hipcc = _hipcc()
    os.makedirs(BUILD_DIR, exist_ok=True)
    objs = []
    cmds = []
    for src in SOURCES:
        obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
        objs.append(obj)
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        cmds.append([hipcc, *COMMON_FLAGS, *lang, "-c", os.path.join(CSRC, src), "-o", obj])
    with ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        for fut in [ex.submit(_run, c, verbose) for c in cmds]:
            fut.result()
    fd, tmp = tempfile.mkstemp(prefix="libpa.", suffix=".so.tmp", dir=HERE)
    os.close(fd)
    try:
        _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs], verbose)
        os.replace(tmp, LIB_PATH)
    finally:
        if os.path.exists(tmp):
            os.unlink(tmp)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
