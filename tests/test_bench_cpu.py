"""The benchmark's own arithmetic and contract, on the CPU: the algorithmic
byte count of a ring all-reduce against a hop-by-hop count, the traffic
figure read from the committed counter summary (and dropped when the kernel
source no longer matches it), the percentile summary, the contention rate
(HOCCL Eq. 1) against a direct integral, and the refusal of more than one
GPU."""
import os
import subprocess
import sys

import numpy as np
import pytest

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _hop_by_hop_bytes(R, count, esize):
    """Sum over the hops of an all-reduce whose last reduce-scatter hop also
    forwards: per element of a chunk, a reduce hop moves 3 operands, the
    forwarding hop 4, an all-gather hop 2; every hop covers all R chunks."""
    chunk = count // R
    total = 0
    for k in range(R - 1):
        total += R * chunk * esize * (4 if k == R - 2 else 3)
    for _ in range(1, R - 1):
        total += R * chunk * esize * 2
    return total


@pytest.mark.parametrize("R,count,esize", [(8, 26214400, 2), (4, 1 << 20, 4), (32, 8 << 20, 4), (2, 64, 2)])
def test_ring_bytes_matches_a_hop_by_hop_count(R, count, esize):
    assert bench.ring_bytes(R, count, esize, fused=True) == _hop_by_hop_bytes(R, count, esize)
    # without the forwarding hop: R-1 reduce hops and R-1 copy hops
    assert bench.ring_bytes(R, count, esize, fused=False) == count * esize * (3 + 2) * (R - 1)


def test_bucket_bytes_figure():
    assert bench.ring_bytes(8, 26214400, 2) == 1_782_579_200


def test_measured_traffic_follows_the_kernel_source(tmp_path, monkeypatch):
    got = bench.measured_traffic()
    assert got is not None and abs(got - 157_286_400) / 157_286_400 < 0.01
    assert bench.measured_traffic("copy_hop_traffic_bytes_per_launch") is not None
    changed = tmp_path / "ccr_kernels.hip"
    changed.write_bytes(open(bench.KERNELS, "rb").read() + b"\n// edited\n")
    monkeypatch.setattr(bench, "KERNELS", str(changed))
    assert bench.measured_traffic() is None


def test_percentiles():
    p = bench.percentiles([5.0, 1.0, 3.0, 2.0, 4.0])
    assert p == {"median_ms": 3.0, "p10_ms": 1.4, "p90_ms": 4.6, "n": 5}
    assert bench.percentiles(np.full(20, 0.25))["median_ms"] == 0.25


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def _contention_brute(intervals, window, n_cu, steps=20000):
    dt = window / steps
    held = 0.0
    for i in range(steps):
        t = (i + 0.5) * dt
        held += min(n_cu, sum(cu for s, e, cu in intervals if s <= t < e)) * dt
    return held / (n_cu * window)


def test_contention_rate_matches_a_direct_integral():
    rng = np.random.default_rng(3)
    for _ in range(20):
        iv = []
        for _ in range(rng.integers(0, 12)):
            s = rng.uniform(-2.0, 11.0)
            iv.append((s, s + rng.uniform(0.01, 4.0), int(rng.integers(1, 300))))
        got = bench.contention_rate(iv, 10.0, 256)
        assert abs(got - _contention_brute(iv, 10.0, 256)) < 2e-3
    assert bench.contention_rate([], 5.0, 256) == 0.0
    # one kernel holding every CU for the whole window, another on top: capped at 1
    assert bench.contention_rate([(0.0, 5.0, 256), (1.0, 2.0, 64)], 5.0, 256) == pytest.approx(1.0)
    # half the CUs for half the window
    assert bench.contention_rate([(2.5, 9.0, 128)], 5.0, 256) == pytest.approx(0.25)


def test_slowdown_summary_names_every_full_cu_run_apart():
    runs = [{"copy_mode": "kernel", "dma_engines": None},
            {"copy_mode": "sdma", "dma_engines": "all"},
            {"copy_mode": "sdma", "dma_engines": 2},
            {"copy_mode": "sdma", "dma_engines": "all", "dma_deadline": {"deadline_us": 2900}}]
    keys = [bench.slowdown_key(r) for r in runs]
    assert keys == ["kernel", "sdma", "sdma_2_engines", "sdma_deadline"]
