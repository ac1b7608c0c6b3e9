"""Build the QSA HIP library (``lib/libqsa.so``) for gfx950 with hipcc.

Usage: ``python -m block_sparse_long_compress_amd.build`` (or call
:func:`build`). Every call recompiles all sources; objects go to
``_build/`` next to this file and the shared library to ``lib/``.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD_DIR = os.path.join(HERE, "_build")
LIB_DIR = os.path.join(HERE, "lib")
LIB_PATH = os.path.join(LIB_DIR, "libqsa.so")

SOURCES = [
    "qsa_api.cpp",
    "qsa_compress.hip",
    "qsa_select.hip",
    "qsa_attn_decode.hip",
    "qsa_attn_prefill.hip",
    "qsa_attn_f32.hip",
    "qsa_decode_step.hip",
    "qsa_indexer.hip",
    "qsa_kv_q8.hip",
    "qsa_noalloc.hip",
]

ARCH = "gfx950"


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    path = os.path.join(rocm, "bin", "hipcc")
    return path if os.path.exists(path) else (shutil.which("hipcc") or "hipcc")


def compile_flags() -> list[str]:
    return [
        "-x", "hip", "-std=c++20", "-O3", "-fPIC", f"--offload-arch={ARCH}",
        # packed fp32 VALU ops stay off: plain scalar/float2 code only
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
        "-I", os.path.join(HERE, "..", "include"),
    ]


# Per-source flags. The prefill attention never holds a NaN (masked scores
# are -inf, and every difference of offsets is guarded), so its max
# reductions need no NaN-quieting copies of their inputs.
EXTRA_FLAGS = {"qsa_attn_prefill.hip": ["-fno-honor-nans"]}


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *compile_flags(), *EXTRA_FLAGS.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    """Compile every source and link ``lib/libqsa.so``; returns the library path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    os.makedirs(LIB_DIR, exist_ok=True)
    jobs = min(len(SOURCES), max(1, min(8, os.cpu_count() or 1)))
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp, *objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, LIB_PATH)
    if verbose:
        print(f"built {LIB_PATH}")
    return LIB_PATH


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
