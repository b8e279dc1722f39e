"""Build the C consumer test program (a plain C user of libccr's C ABI,
checked against the C oracle) next to its source:

    python tests/c_consumer/build.py

It links the in-tree libccr.so and libccr_oracle.so and ROCm's own HIP
runtime, so it runs without Python or PyTorch."""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
SRC = os.path.join(HERE, "ccr_c_consumer.c")
EXE = os.path.join(HERE, "ccr_c_consumer")


def build() -> str:
    cmd = ["gcc", "-std=c11", "-O2", "-Wall", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
           "-I" + os.path.join(ROOT, "include"), SRC, "-o", EXE,
           "-L" + os.path.join(ROOT, "collective_communication_reduce_amd"), "-lccr",
           "-L" + os.path.join(ROOT, "oracle"), "-lccr_oracle", "-L/opt/rocm/lib", "-lamdhip64",
           "-Wl,--disable-new-dtags,-rpath,$ORIGIN/../../collective_communication_reduce_amd:"
           "$ORIGIN/../../oracle:/opt/rocm/lib"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"building the C consumer failed:\n{r.stdout}{r.stderr}")
    return EXE


if __name__ == "__main__":
    print(build())
