"""Build libkvc.so in-tree with hipcc for gfx950 (no torch extension machinery).

    python -m kv_cache_compression_pool_amd._build
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OUT = os.path.join(PKG, "libkvc.so")
BUILD_DIR = os.path.join(PKG, "_build")

SOURCES = ["kvc_api.cpp", "kvc_pool16.hip", "kvc_c128.hip", "kvc_diag.hip"]

# Packed-fp32 instructions are disabled on purpose: plain fp32 VALU code only.
HIP_FLAGS = ["--offload-arch=gfx950", "-O3", "-fPIC", "-std=c++17", "-Wall",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-I", INCLUDE, "-I", CSRC]


def hipcc() -> str:
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        raise RuntimeError("hipcc not found; the HIP library cannot be built")
    return exe


def build(verbose: bool = False) -> str:
    """Compile every source and link libkvc.so (always rebuilds)."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    objs = []
    for src in SOURCES:
        obj = os.path.join(BUILD_DIR, src + ".o")
        cmd = [hipcc(), *HIP_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        # The host pass does not know the packed-fp32 feature and says so.
        msgs = [ln for ln in (r.stdout + r.stderr).splitlines()
                if "packed-fp32-ops" not in ln]
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n" + "\n".join(msgs))
        if verbose and msgs:
            print("\n".join(msgs))
        objs.append(obj)
    tmp = OUT + ".tmp"
    subprocess.check_call([hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", *objs,
                           "-o", tmp])
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
