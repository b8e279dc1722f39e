"""The C ABI from plain C: a program with no Python and no PyTorch (HIP's own
runtime from ROCm) runs the ring calls, the staged ring shift and the
uniform element all-to-all through libccr, with kernel and SDMA copies, and
compares every byte with the C oracle (tests/c_consumer/ccr_c_consumer.c,
built by __graft_entry__.build())."""
import os
import subprocess

import pytest

from gpu_helpers import say

pytestmark = pytest.mark.gpu

EXE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c_consumer", "ccr_c_consumer")


def test_c_program_through_the_c_abi():
    assert os.path.exists(EXE), f"{EXE} is missing: build it with __graft_entry__.build()"
    say("C consumer program")
    r = subprocess.run([EXE], capture_output=True, text=True, timeout=240)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    lines = r.stdout.splitlines()
    assert lines[-1] == "c consumer: ok", r.stdout[-3000:]
    assert sum(1 for l in lines if l.endswith(": ok") and "c consumer" not in l) == 2 * (5 * 2 * 2 + 2)
