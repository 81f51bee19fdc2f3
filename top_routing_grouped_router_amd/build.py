"""Build the HIP library of the MoE layer for gfx950: csrc/*.hip -> lib/libmoe_mi355x.so.

Each translation unit compiles in parallel with hipcc to an object under _build/, then one
shared library is linked. The library exports only the C ABI of include/moe_mi355x.h.
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
LIBDIR = os.path.join(PKG, "lib")
LIBNAME = "libmoe_mi355x.so"
ARCH = "gfx950"

HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"

CFLAGS = [
    "-O3", "-std=c++17", f"--offload-arch={ARCH}", "-fPIC", "-fvisibility=hidden",
    "-Wall", "-Wno-unused-function",
    # keep the compiler from emitting packed fp32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def lib_path() -> str:
    return os.path.join(LIBDIR, LIBNAME)


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # hipcc's host pass warns that it does not know the packed-fp32 feature: harmless.
    out = "\n".join(line for line in r.stdout.splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in line)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(verbose: bool = False, jobs: int | None = None) -> str:
    os.makedirs(BUILD, exist_ok=True)
    os.makedirs(LIBDIR, exist_ok=True)
    srcs = sorted(f for f in os.listdir(CSRC) if f.endswith(".hip"))
    objs = [os.path.join(BUILD, os.path.splitext(f)[0] + ".o") for f in srcs]

    def compile_one(pair):
        src, obj = pair
        return _run([HIPCC, *CFLAGS, "-c", os.path.join(CSRC, src), "-o", obj])

    jobs = jobs or min(len(srcs), max(1, (os.cpu_count() or 4)))
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        outs = list(ex.map(compile_one, zip(srcs, objs)))
    tmp = lib_path() + ".tmp"
    outs.append(_run([HIPCC, "-shared", f"--offload-arch={ARCH}", "-fPIC", "-o", tmp, *objs]))
    os.replace(tmp, lib_path())
    if verbose:
        for o in outs:
            if o.strip():
                print(o)
    return lib_path()


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
