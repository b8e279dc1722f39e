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
    for i in range(len(bench.KERNELS)):  # an edit of any of the kernel sources
        changed = tmp_path / f"edited_{i}"
        changed.write_bytes(open(bench.KERNELS[i], "rb").read() + b"\n// edited\n")
        monkeypatch.setattr(bench, "KERNELS", bench.KERNELS[:i] + [str(changed)] + bench.KERNELS[i + 1:])
        assert bench.measured_traffic() is None
        monkeypatch.undo()


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


def test_ci95_against_scipy_and_a_normal_sample():
    from scipy import stats
    rng = np.random.default_rng(1)
    x = rng.normal(2.0, 0.5, 15)
    m, lo, hi = bench.ci95(x)
    want = stats.t.interval(0.95, 14, loc=x.mean(), scale=stats.sem(x))
    assert m == pytest.approx(x.mean()) and (lo, hi) == pytest.approx(want)
    d, lo, hi = bench.diff_ci95(x + 1.0, x)
    assert d == pytest.approx(1.0) and lo < 1.0 < hi
    assert bench.ci95([3.0]) == (3.0, 3.0, 3.0)


def test_pareto_keeps_only_undominated_points():
    pts = [("a", 19.0, 0.7), ("b", 30.0, 0.2), ("c", 24.0, 1.5), ("d", 26.0, 7.0), ("e", 19.0, 0.9)]
    assert bench.pareto(pts) == ["a", "b"]
    assert bench.pareto([("x", 1.0, 1.0)]) == ["x"]


def _run(mode, B, eng, pairs, coll, **kw):
    r = {"copy_mode": mode, "cu_budget": B, "dma_engines": eng,
         "dma_sync": "host_func" if mode == "sdma" else None, "pairs_pct": list(pairs),
         "slowdown_mean_pct": float(np.mean(pairs)), "collectives_under_load_ms": coll, **kw}
    r["label"] = bench.run_label(r)
    return r


def test_sdma_verdict_compares_equal_budgets_and_matched_times():
    rng = np.random.default_rng(2)
    noise = lambda m: m + rng.normal(0, 0.05, 15)  # noqa: E731
    runs = [_run("kernel", 256, None, noise(0.6), 19.0), _run("kernel", 16, None, noise(7.0), 26.5),
            _run("sdma", 256, "all", noise(1.6), 21.6), _run("sdma", 16, "all", noise(9.0), 26.4),
            _run("sdma", 256, 2, noise(0.2), 30.0), _run("sdma", 256, 4, noise(1.2), 26.0),
            _run("sdma", 256, "all", noise(12.0), 15.0, dma_sync="stream_flags")]
    v = bench.sdma_verdict(runs)
    eq = {e["cu_budget"]: e for e in v["equal_budget"]}
    assert set(eq) == {256, 16}
    assert eq[256]["sdma_higher"] and not eq[256]["sdma_lower"] and v["target_sdma_lower_at_full_cus"] is False
    m = {x["sdma"]: x for x in v["matched_time"]}
    # SDMA on 4 engines (26.0 ms) is matched with kernel copies at 16 CUs (26.5 ms) and beats them
    assert m["sdma/B256/E4"]["kernel"] == "kernel/B16" and m["sdma/B256/E4"]["sdma_lower"]
    assert v["sdma_lower_at_some_matched_time"]
    assert "sdma/B256/Eall/flags" not in str(v)  # flag-handshake runs stay out of the comparison
    assert v["pareto"] == ["kernel/B256", "sdma/B256/E2"]
    c = bench.compact_verdict({"verdict": v})
    assert len(json_dumps(c)) < 1500 and c["sdma_lower_at_full_cus"] is False


def json_dumps(o):
    import json
    return json.dumps(o)


def test_contention_from_trace_rows():
    def row(name, b, e, grid, wg=256):
        return {"Kernel_Name": name, "Start_Timestamp": str(b), "End_Timestamp": str(e),
                "Grid_Size_X": str(grid * wg), "Workgroup_Size_X": str(wg)}
    rows = [row("void ccr::pieces_kernel<...>", 0, 500, 6400),  # before the window: ignored
            row("at::cuda::sleep(long)", 1000, 2000, 1),
            row("Cijk_gemm", 2000, 12000, 1024), row("Cijk_gemm", 12000, 22000, 1024),
            row("void ccr::pieces_kernel<...>", 5000, 7000, 6400),   # 256 CUs for 2 us
            row("void ccr::pieces_kernel<...>", 20000, 25000, 64)]   # 64 CUs, 2 us inside the window
    got = bench.contention_from_trace(rows)
    want = (256 * 2000 + 64 * 2000) / (256 * 20000)
    assert got["interval_bound"] == pytest.approx(want, abs=1e-4)
    assert got["compute_kernels"] == 2 and got["collective_kernels"] == 2
    # torch's GPU sleep is named spin_kernel on this stack
    rows[1]["Kernel_Name"] = "at::cuda::(anonymous namespace)::spin_kernel(long)"
    assert bench.contention_from_trace(rows)["compute_kernels"] == 2
    # the work-based estimate: each kernel needs 500 ns alone; the second one
    # lies 2/5 inside the window
    got = bench.contention_from_trace(rows, alone={"void ccr::pieces_kernel<...>": 500})
    want = (500 * 256 + 500 * (2000 / 5000) * 64) / (256 * 20000)
    assert got["work_estimate"] == pytest.approx(want, abs=1e-4)
    assert bench.kernel_means(rows)["Cijk_gemm"] == pytest.approx(10000)


def test_reduce_hops_by_position():
    iv = np.array([[0.0, 0.033, 256], [0.04, 0.064, 256], [0.07, 0.094, 256]] * 2)
    out = bench.reduce_hops_by_position(iv, 157286400, 2)
    assert out["first_hop"]["mean_launch_us"] == pytest.approx(33.0)
    assert out["later_hops"]["mean_launch_us"] == pytest.approx(24.0)
    assert out["first_hop"]["bound"] == "hbm" and out["later_hops"]["bound"] == "hbm+mall"
    assert bench.reduce_hops_by_position(iv, 1, 4) is None
