"""The stream/proxy hand-over state of the SDMA path, checked on the CPU.

``csrc/ccr_handoff.h`` holds the host-side state machines that tie an SDMA
job to a stream: the host-function gate (a block shared by the proxy's job
and the stream's callback, freed by whichever lets go last) and the flag
words (a request and a done word per slot, increasing sequence numbers, a
wait that passes once done >= the job's number).  ``handoff_check.cpp``
drives them from host threads that stand in for the stream: release before
and after arrival, abandonment racing arrival, slot reuse while an older
wait is pending, a late stream after abandonment, and many streams at once.
It is built with g++ under AddressSanitizer + UndefinedBehaviorSanitizer and
again under ThreadSanitizer, so a use after free or a data race fails the
test.  No GPU is used."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.parametrize("sanitize", ["address,undefined", "thread"])
def test_handoff_state_machines(tmp_path, sanitize):
    if not shutil.which("g++"):
        pytest.skip("g++ is not installed")
    exe = tmp_path / "handoff_check"
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-pthread", f"-fsanitize={sanitize}",
           "-fno-omit-frame-pointer", os.path.join(HERE, "handoff_check.cpp"), "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0 and "sanitizer" in (r.stderr or "").lower():
        pytest.skip(f"the {sanitize} sanitizer runtime is not available: {r.stderr[-300:]}")
    assert r.returncode == 0, r.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:verify_asan_link_order=0",
               TSAN_OPTIONS="halt_on_error=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "handoff: ok" in r.stdout
