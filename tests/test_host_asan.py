"""The C ABI's host code under AddressSanitizer (CPU only).

tests/asan/abi_host_driver.cpp calls every entry point with arguments the host validation
rejects, and the pure host queries (defaults, parameter counts, capacities, workspace sizes,
messages) over a grid of shapes; none of those calls reaches a HIP call. The library sources
are compiled with the sanitizer on the host side only (-Xarch_host), linked with the driver
and run: an out-of-bounds access, use after free or leak in the host code fails the test.
"""
import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "top_routing_grouped_router_amd", "csrc")
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
FLAGS = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
         "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}"]


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not found")
def test_abi_host_code_under_address_sanitizer(tmp_path):
    srcs = sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))
    srcs.append(os.path.join(ROOT, "tests", "asan", "abi_host_driver.cpp"))

    def compile_one(src):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        r = subprocess.run([HIPCC, *FLAGS, "-x", "hip", "-c", src, "-o", obj], capture_output=True, text=True)
        assert r.returncode == 0, r.stdout + r.stderr
        return obj

    with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(compile_one, srcs))
    exe = str(tmp_path / "abi_host_driver")
    r = subprocess.run([HIPCC, "--offload-arch=gfx950", "-Xarch_host", "-fsanitize=address", *objs, "-o", exe],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:exitcode=86")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0 and "all checks passed" in r.stdout, r.stdout + r.stderr
