"""The C ABI layer's host code (planners, validation) built with
AddressSanitizer against launcher stubs and fuzzed with random batches on the
CPU: exact and tight capacities, padding on and off."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(ROOT, "kv_cache_compression_pool_amd", "csrc")
INC = os.path.join(ROOT, "include")


def _tool(name):
    return shutil.which(name) or (f"/opt/rocm/bin/{name}" if os.path.exists(f"/opt/rocm/bin/{name}")
                                  else None)


@pytest.mark.skipif(not (_tool("hipcc") and shutil.which("g++")), reason="needs hipcc and g++")
def test_planners_under_address_sanitizer(tmp_path):
    hipcc, out = _tool("hipcc"), str(tmp_path)
    inc = ["-I", INC, "-I", CSRC]
    # host code only: the sanitizer flag applies to the host pass alone
    subprocess.check_call([hipcc, "-std=c++17", "-O1", "-g", "-fPIC", "-Xarch_host",
                           "-fsanitize=address", *inc, "-c", os.path.join(CSRC, "kvc_api.cpp"),
                           "-o", f"{out}/api.o"], stderr=subprocess.DEVNULL)
    for src, obj, extra in (("launcher_stubs.cpp", "stubs.o", ["-I", "/opt/rocm/include",
                                                               "-D__HIP_PLATFORM_AMD__"]),
                            ("planner_fuzz.cpp", "fuzz.o", [])):
        subprocess.check_call(["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address", *inc,
                               *extra, "-c", os.path.join(HERE, "host_asan", src), "-o",
                               f"{out}/{obj}"])
    subprocess.check_call(["g++", "-no-pie", "-fsanitize=address", f"{out}/fuzz.o", f"{out}/api.o",
                           f"{out}/stubs.o", "-L/opt/rocm/lib", "-lamdhip64",
                           "-Wl,-rpath,/opt/rocm/lib", "-o", f"{out}/fuzz"])
    r = subprocess.run([f"{out}/fuzz", "5000"], capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "ok" in r.stdout
