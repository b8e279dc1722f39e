"""Build libccr.so (the C-ABI library) in place with hipcc for gfx950.

    python collective_communication_reduce_amd/build.py

The library is built in-tree next to this file so it travels with the
source tree; nothing is installed.
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
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libccr.so")
SOURCES = ["ccr_api.cpp", "ccr_dma.cpp", "ccr_schedule.cpp", "ccr_kernels.hip", "ccr_ring.hip",
           "ccr_moe_kernels.hip", "ccr_scratch.hip"]
# Per-source additions: the ring-hop kernels take their leading scalar
# arguments preloaded into registers (gfx950 kernel-argument preloading), so
# a workgroup's first scalar memory access is the load of its base addresses.
SOURCE_FLAGS = {"ccr_ring.hip": ["-mllvm", "-amdgpu-kernarg-preload-count=16"]}
ARCH = "gfx950"

# -packed-fp32-ops keeps the compiler from emitting packed fp32 arithmetic;
# denormals are kept (IEEE behaviour, no flush) and no FMA contraction is
# allowed, so fp32 sums are plain IEEE round-to-nearest-even adds.
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-ffp-contract=off", "-fno-gpu-flush-denormals-to-zero", "-fno-fast-math",
    "-I" + os.path.join(ROOT, "include"),
]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found; the HIP library cannot be built")


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    cc = hipcc()

    def compile_one(src):
        obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
        cmd = [cc, *FLAGS, *SOURCE_FLAGS.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        noise = "is not a recognized feature for this target"
        err = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if noise not in l)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{err}")
        if verbose and err.strip():
            print(err, file=sys.stderr)
        return obj

    with ThreadPoolExecutor(len(SOURCES)) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = LIB + ".tmp"
    # libhsa-runtime64 (SDMA engine copies): resolved at load time to the HSA
    # runtime already in the process (torch's), like libamdhip64.  The roctx
    # library marks each entry point for rocprofv3's marker trace.
    r = subprocess.run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs,
                        "-L/opt/rocm/lib", "-lhsa-runtime64", "-lrocprofiler-sdk-roctx"],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link of libccr.so failed:\n{r.stdout}{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
