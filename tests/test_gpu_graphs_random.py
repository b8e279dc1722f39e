"""Seeded random sweep of ring calls captured into a HIP graph by the caller
and replayed: kernel copies and per-hop accumulation (the calls that may be
captured), 1-64 ranks, ragged sizes, fp32 and bf16, all-reduce,
reduce-scatter, all-gather and reduce-scatter followed by all-gather, 1-5
slices with or without overlap (whose side streams join the capture through
the call's fork and join events).  Each graph is replayed three times, the
inputs restored before each replay and eager calls of the same context on
other buffers run between replays; every replay is compared bit for bit with
the oracle.  The cases are fixed by the seed."""
import numpy as np
import pytest

import oracle
import workloads
from gpu_helpers import say, to_dev, to_host, torch_cuda

pytestmark = pytest.mark.gpu

N_CASES = 150


def _cases(seed=9191):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(N_CASES):
        R = int(rng.choice([1, 2, 3, 4, 5, 8, 9, 13, 16, 32, 64]))
        n = int(10 ** rng.uniform(0, 5))
        dt = "bf16" if rng.random() < 0.5 else "f32"
        op = str(rng.choice(["allreduce", "allreduce", "rs", "ag", "rs_ag"]))
        cfg = {"slices": int(rng.integers(1, 6))}
        if rng.random() < 0.4:
            cfg["overlap"] = True
        out.append((i, R, n, dt, op, cfg))
    return out


CASES = _cases()


@pytest.fixture(scope="module")
def ccr_mod():
    torch_cuda()
    import collective_communication_reduce_amd as ccr
    return ccr


def _call(ccr, ctx, op, ts):
    if op == "allreduce":
        ccr.ccr_allreduce(ctx, ts)
    elif op == "rs":
        ccr.ccr_reduce_scatter(ctx, ts)
    elif op == "ag":
        ccr.ccr_all_gather(ctx, ts)
    else:
        ccr.ccr_reduce_scatter(ctx, ts)
        ccr.ccr_all_gather(ctx, ts)


def _expected(xs, op, S):
    if op == "allreduce":
        return oracle.ring_allreduce(xs, S=S)
    if op == "rs":
        return oracle.ring_reduce_scatter(xs, S=S)
    if op == "ag":
        return oracle.ring_all_gather(xs, S=S)
    return oracle.ring_all_gather(oracle.ring_reduce_scatter(xs, S=S), S=S)


@pytest.mark.parametrize("case", CASES, ids=[f"case{c[0]}" for c in CASES])
def test_random_captured_ring_case(ccr_mod, case):
    import torch
    i, R, n, dt, op, cfg = case
    say(f"random captured case {i}: R={R} n={n} {dt} {op} {cfg}")
    xs = workloads.random_buffers(R, n, dt, seed=7000 + i, dist="normal", scale=1.0)
    want = _expected(xs, op, cfg["slices"])
    with ccr_mod.Context(0, ccr_mod.Config(**cfg)) as c:
        src = [to_dev(x) for x in xs]
        bufs = [t.clone() for t in src]
        other = [t.clone() for t in src]
        _call(ccr_mod, c, op, other)  # eager first call: side streams and events exist
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        with torch.cuda.graph(g, stream=s):
            _call(ccr_mod, c, op, bufs)
            if R == 1:  # the call enqueues nothing: keep the graph non-empty
                bufs[0].mul_(1)
        for rep in range(3):
            for b, t in zip(bufs, src):
                b.copy_(t)
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            for q in range(R):
                got = to_host(bufs[q])
                if got.tobytes() != want[q].tobytes():
                    bad = np.nonzero(got != want[q])[0]
                    raise AssertionError(f"case {i} replay {rep}: rank {q} differs at {bad.size} "
                                         f"elements, first {bad[:5]}")
            for b, t in zip(other, src):  # eager work of the same context between replays
                b.copy_(t)
            _call(ccr_mod, c, op, other)
            torch.cuda.synchronize()
        for q in range(R):
            assert to_host(other[q]).tobytes() == want[q].tobytes(), f"case {i} eager rank {q}"
        del g
