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
