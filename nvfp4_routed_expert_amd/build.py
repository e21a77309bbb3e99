"""Build libnvfp4moe.so from the HIP sources in csrc/ for gfx950.

Every translation unit is compiled by hipcc for gfx950 only and linked into
one shared library next to this file.  Usage: ``python -m
nvfp4_routed_expert_amd.build`` (or ``build()`` from Python).
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD_DIR = os.path.join(os.path.dirname(HERE), "_build")
LIB_NAME = "libnvfp4moe.so"
LIB_PATH = os.path.join(HERE, LIB_NAME)
ARCH = "gfx950"

COMMON_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17",
    # packed fp32 VALU forms stay off: plain scalar fp32 only
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
]
# Quantisation must round every fp32 step on its own (no FMA contraction).
PER_FILE_FLAGS = {"quant.hip": ["-ffp-contract=off"]}


def hipcc() -> str:
    cand = os.environ.get("HIPCC") or shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(cand):
        raise RuntimeError("hipcc not found; the HIP library cannot be built")
    return cand


def sources():
    return sorted(f for f in os.listdir(CSRC) if f.endswith(".hip"))


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, src.replace(".hip", ".o"))
    cmd = [hipcc(), *COMMON_FLAGS, *PER_FILE_FLAGS.get(src, []), "-c",
           os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"compiling {src} failed:\n{' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    noise = ("packed-fp32-ops", "argument unused")
    warn = "\n".join(l for l in res.stderr.splitlines() if l and not any(n in l for n in noise))
    if warn.strip():
        print(f"[build] {src}:\n{warn}", file=sys.stderr)
    return obj


def build(verbose: bool = True) -> str:
    """Compile every csrc/*.hip for gfx950 and link the shared library."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = sources()
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"linking failed:\n{' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, LIB_PATH)
    if verbose:
        print(f"[build] {LIB_PATH} ({len(objs)} objects)")
    return LIB_PATH


if __name__ == "__main__":
    build()
