"""Stream semantics of the collectives on the GPU: a call keeps its place in
the caller's stream order (work enqueued before it on that stream is seen,
work enqueued after it sees the results), in every copy / overlap / budget
mode, and contexts on different streams do not disturb each other.  Results
are checked bit for bit against the oracle."""
import numpy as np
import pytest

import oracle
import workloads
from gpu_helpers import say, to_dev, to_host, torch_cuda

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ccr_mod():
    torch_cuda()
    import collective_communication_reduce_amd as ccr
    return ccr


MODES = [dict(), dict(overlap=True, slices=3), dict(copy_mode="sdma"),
         dict(copy_mode="sdma", slices=2), dict(cu_budget=32, slices=2, overlap=True),
         dict(bf16_acc="fp32_partials", overlap=True, slices=2)]

# ~10 ms at the GPU's clock: the producer is still pending when the
# collective is enqueued.
SLEEP_CYCLES = 20_000_000


@pytest.mark.parametrize("mode", MODES, ids=lambda m: "-".join(f"{k}={v}" for k, v in m.items()) or "default")
@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_call_keeps_its_place_in_the_stream(ccr_mod, mode, dt):
    """Producer copies on the caller's stream (behind a GPU sleep), the
    all-reduce, then a consumer copy and an overwrite on the same stream,
    with no host synchronisation in between."""
    import torch
    R, n = 5, 2 * 65536 + 37
    xs = workloads.random_buffers(R, n, dt, seed=404, dist="normal", scale=1e-2)
    acc = mode.get("bf16_acc", "per_hop") if dt == "bf16" else "per_hop"
    expect = oracle.ring_allreduce(xs, S=1, bf16_acc=acc)
    say(f"stream order {dt} R={R} n={n} mode={mode}")
    src = [to_dev(x) for x in xs]
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    with ccr_mod.Context(0, ccr_mod.Config(**mode)) as c:
        bufs = [torch.zeros_like(t) for t in src]
        torch.cuda.synchronize()
        with torch.cuda.stream(s):
            torch.cuda._sleep(SLEEP_CYCLES)
            for b, t in zip(bufs, src):
                b.copy_(t)
            ccr_mod.ccr_allreduce(c, bufs, stream=s)
            out = [b.clone() for b in bufs]
            for b in bufs:
                b.fill_(7)
        s.synchronize()
        for q in range(R):
            assert to_host(out[q]).tobytes() == expect[q].tobytes(), f"rank {q}"


@pytest.mark.parametrize("modes", [(dict(), dict(copy_mode="sdma")),
                                   (dict(overlap=True, slices=2), dict(cu_budget=64)),
                                   (dict(bf16_acc="fp32_partials"), dict(bf16_acc="fp32_partials"))],
                         ids=["kernel+sdma", "overlap+budget", "partials+partials"])
def test_two_contexts_on_two_streams(ccr_mod, modes):
    """Two contexts, two caller streams, two all-reduces of different shapes
    enqueued back to back before any synchronisation."""
    import torch
    cases = [(4, 3 * 65536 + 5, 11), (8, 65536 * 2 + 3, 12)]
    ins = [workloads.random_buffers(R, n, "bf16", seed=sd, dist="normal", scale=1e-3)
           for R, n, sd in cases]
    exp = [oracle.ring_allreduce(x, S=1, bf16_acc=m.get("bf16_acc", "per_hop"))
           for x, m in zip(ins, modes)]
    say(f"two contexts on two streams {modes}")
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    ctxs = [ccr_mod.Context(0, ccr_mod.Config(**m)) for m in modes]
    try:
        dev = [[to_dev(x) for x in xs] for xs in ins]
        torch.cuda.synchronize()
        for rep in range(3):  # repeated: the second call of each context reuses its scratch
            if rep:
                for d, xs in zip(dev, ins):
                    for t, x in zip(d, xs):
                        t.copy_(to_dev(x))
                torch.cuda.synchronize()
            for c, d, s in zip(ctxs, dev, streams):
                ccr_mod.ccr_allreduce(c, d, stream=s)
            torch.cuda.synchronize()
            for d, e in zip(dev, exp):
                for q, t in enumerate(d):
                    assert to_host(t).tobytes() == e[q].tobytes(), f"rep {rep} rank {q}"
    finally:
        for c in ctxs:
            c.close()


def _kfd_queues():
    """Hardware queues the kernel driver lists for this process, or None
    where its per-process sysfs directory cannot be read."""
    import os
    d = f"/sys/class/kfd/kfd/proc/{os.getpid()}/queues"
    try:
        return len(os.listdir(d))
    except OSError:
        return None


def test_contexts_hold_no_hardware_queue_until_a_call_needs_one(ccr_mod):
    """Ten contexts making kernel-copy calls that need no second stream hold
    no side stream (and, where the driver lists the process's hardware
    queues, add none); a CU budget makes the budgeted stream with the
    context; an overlapped all-gather or an SDMA one over several slices
    makes the second stream on its first call; the graph cache captures on a
    plain stream.  Results stay those of the oracle."""
    import torch
    R, n = 8, 65536 + 8
    xs = workloads.random_buffers(R, n, "f32", seed=21, dist="normal")
    ref = oracle.ring_allreduce(xs, S=1)
    say("side streams are made on demand")
    ts = [to_dev(x) for x in xs]
    torch.cuda.synchronize()
    q0 = _kfd_queues()
    ctxs = [ccr_mod.Context(0, ccr_mod.Config(graph_cache=False)) for _ in range(10)]
    try:
        for c in ctxs:
            for t, x in zip(ts, xs):
                t.copy_(to_dev(x))
            ccr_mod.ccr_allreduce(c, ts)
            ccr_mod.ccr_sendrecv_batch(c, ts[:2], ts[2:4])
            torch.cuda.synchronize()
            assert ccr_mod.ccr_ctx_streams(c) == (0, 0)
        q1 = _kfd_queues()
        if q0 is not None and q1 is not None:
            assert q1 == q0, (q0, q1)
    finally:
        for c in ctxs:
            c.close()
    cases = [(dict(cu_budget=16), (1, 0), (1, 0)), (dict(overlap=True, slices=2), (0, 0), (1, 0)),
             (dict(copy_mode="sdma", slices=2), (0, 0), (1, 0)), (dict(copy_mode="sdma"), (0, 0), (0, 0)),
             (dict(cu_budget=16, overlap=True, slices=2), (1, 0), (2, 0))]
    for cfg, at_create, after_call in cases:
        with ccr_mod.Context(0, ccr_mod.Config(graph_cache=False, **cfg)) as c:
            assert ccr_mod.ccr_ctx_streams(c) == at_create, cfg
            for t, x in zip(ts, xs):
                t.copy_(to_dev(x))
            ccr_mod.ccr_allreduce(c, ts)
            torch.cuda.synchronize()
            assert ccr_mod.ccr_ctx_streams(c) == after_call, cfg
            for q, t in enumerate(ts):
                assert to_host(t).tobytes() == ref[q].tobytes(), f"{cfg} rank {q}"
    small = [to_dev(x[:4096]) for x in xs]
    with ccr_mod.Context(0) as c:  # graph cache: captured on the second call
        for _ in range(3):
            ccr_mod.ccr_allreduce(c, small)
        torch.cuda.synchronize()
        assert ccr_mod.ccr_ctx_streams(c) == (0, 1)
        assert ccr_mod.ccr_graph_cache_stats(c)[1] >= 1
