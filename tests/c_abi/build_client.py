"""Build the plain C client of libkvc (kvc_c_client.c) next to its source.

    python -m tests.c_abi.build_client

gcc compiles it as C11 against include/kvc.h and the HIP runtime headers and
links libkvc.so (found at run time through a relative rpath) and libamdhip64.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
SRC = os.path.join(HERE, "kvc_c_client.c")
OUT = os.path.join(HERE, "kvc_c_client")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build(out: str = OUT) -> str:
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        raise RuntimeError("no C compiler found for the C client")
    lib_dir = os.path.join(ROOT, "kv_cache_compression_pool_amd")
    if not os.path.exists(os.path.join(lib_dir, "libkvc.so")):
        raise RuntimeError("libkvc.so must be built before the C client")
    cmd = [cc, "-std=c11", "-O2", "-Wall", "-Wextra", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROCM, "include"), "-I", os.path.join(ROOT, "include"), SRC,
           "-L", lib_dir, "-l:libkvc.so", "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
           "-Wl,-rpath,$ORIGIN/../../kv_cache_compression_pool_amd",
           "-Wl,-rpath," + os.path.join(ROCM, "lib"), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("C client build failed:\n" + r.stdout + r.stderr)
    return out


if __name__ == "__main__":
    print(build())
