"""Contexts used from several host threads at once, one context per thread
(each call releases Python's lock while the library runs): every thread on
its own stream and in its own mode (kernel copies, SDMA copies, overlap,
fp32 partials) makes repeated all-reduces and reduce-scatter + all-gather
pairs, each result bit for bit against the oracle."""
import threading

import numpy as np
import pytest

import oracle
import workloads
from gpu_helpers import say, to_dev, to_host, torch_cuda

pytestmark = pytest.mark.gpu

WORKERS = [(4, 100003, "f32", {}), (8, 65536 + 9, "bf16", {"copy_mode": "sdma"}),
           (5, 4099, "bf16", {"overlap": True, "slices": 3}),
           (16, 30011, "bf16", {"bf16_acc": "fp32_partials"})]


@pytest.fixture(scope="module")
def ccr_mod():
    torch_cuda()
    import collective_communication_reduce_amd as ccr
    return ccr


def test_contexts_on_separate_host_threads(ccr_mod):
    import torch
    errors, done = [], []
    start = threading.Barrier(len(WORKERS))

    def worker(k, R, n, dt, cfg):
        try:
            xs = workloads.random_buffers(R, n, dt, seed=900 + k, dist="normal", scale=1.0)
            acc = cfg.get("bf16_acc", "per_hop")
            want = oracle.ring_allreduce(xs, S=1, bf16_acc=acc)
            s = torch.cuda.Stream()
            with torch.cuda.stream(s), ccr_mod.Context(0, ccr_mod.Config(**cfg)) as c:
                src = [to_dev(x) for x in xs]
                start.wait(timeout=60)
                for it in range(12):
                    ts = [t.clone() for t in src]
                    if it % 2:
                        ccr_mod.ccr_reduce_scatter(c, ts)
                        ccr_mod.ccr_all_gather(c, ts)
                    else:
                        ccr_mod.ccr_allreduce(c, ts)
                    s.synchronize()
                    for q in range(R):
                        got = to_host(ts[q])
                        if got.tobytes() != want[q].tobytes():
                            bad = np.nonzero(got != want[q])[0]
                            raise AssertionError(f"worker {k} call {it}: rank {q} differs at {bad.size} elements")
            done.append(k)
        except Exception as e:  # reported by the main thread
            errors.append((k, repr(e)))

    say(f"{len(WORKERS)} host threads, one context each: {[w[3] for w in WORKERS]}")
    threads = [threading.Thread(target=worker, args=(k, *w), daemon=True) for k, w in enumerate(WORKERS)]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not errors, errors
    assert sorted(done) == list(range(len(WORKERS)))
