"""HIP graph capture of the collectives.  Calls made of kernel launches only
(the ring with kernel copies and per-hop bf16, with or without side
streams; the kernel-copy all-to-all; the three-stage MoE dispatch and
combine; row permutes; top-K) are captured and
replayed several times, with eager work and synchronisations between the
replays, every replay checked bit for bit against the oracle.  Calls that
depend on context scratch that may be reallocated, on host memory copied at
launch, or on the DMA proxy are refused while the stream is capturing."""
import numpy as np
import pytest

import oracle
import workloads
from gpu_helpers import raw_to_dev, say, to_dev, to_host, torch_cuda

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ccr_mod():
    torch_cuda()
    import collective_communication_reduce_amd as ccr
    return ccr


def _replays(torch, g, reset, check, other):
    for rep in range(4):
        reset()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        check(rep)
        other()  # eager work of the program between replays
        torch.cuda.synchronize()


@pytest.mark.parametrize("mode", [dict(), dict(slices=2), dict(overlap=True, slices=2)],
                         ids=["default", "slices2", "overlap"])
@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_captured_allreduce_replays(ccr_mod, mode, dt):
    import torch
    R, n = 4, 3 * 65536 + 5
    xs = workloads.random_buffers(R, n, dt, seed=77, dist="normal", scale=1e-2)
    expect = oracle.ring_allreduce(xs, S=1)
    say(f"graph allreduce {dt} mode={mode}")
    with ccr_mod.Context(0, ccr_mod.Config(**mode)) as c:
        src = [to_dev(x) for x in xs]
        bufs = [t.clone() for t in src]
        scratch = [t.clone() for t in src]
        ccr_mod.ccr_allreduce(c, bufs)  # warm-up outside the capture
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        with torch.cuda.graph(g, stream=s):
            ccr_mod.ccr_allreduce(c, bufs)

        def reset():
            for b, t in zip(bufs, src):
                b.copy_(t)

        def check(rep):
            for q in range(R):
                assert to_host(bufs[q]).tobytes() == expect[q].tobytes(), f"replay {rep} rank {q}"

        def other():
            for b, t in zip(scratch, src):
                b.copy_(t)
            ccr_mod.ccr_allreduce(c, scratch)

        _replays(torch, g, reset, check, other)
        for q in range(R):  # the eager calls between replays were right too
            assert to_host(scratch[q]).tobytes() == expect[q].tobytes()


def test_captured_alltoall_permute_topk_replays(ccr_mod):
    import torch
    R, row = 4, 48
    rng = np.random.default_rng(5)
    counts = rng.integers(0, 9, (R, R))
    sends = [rng.integers(0, 256, int(counts[r].sum()) * row, dtype=np.uint8) for r in range(R)]
    ref = oracle.alltoall(sends, counts, row)
    T, E, K = 64, 16, 3
    logits = rng.standard_normal((T, E)).astype(np.float32)
    ref_topk = oracle.moe_topk(logits, K)
    nsrc, nrows = 50, 70
    src_rows = rng.integers(0, 256, (nsrc, 32), dtype=np.uint8)
    idx = rng.integers(0, nsrc, nrows).astype(np.int32)
    say("graph alltoall / permute / topk")
    with ccr_mod.Context(0) as c:
        s_d = [raw_to_dev(x) for x in sends]
        r_d = [torch.zeros(max(16, x.size), dtype=torch.uint8, device="cuda") for x in ref]
        d_logits = to_dev(logits)
        d_topk = torch.zeros(T, K, dtype=torch.int32, device="cuda")
        d_src = torch.from_numpy(src_rows).cuda()
        d_idx = torch.from_numpy(idx).cuda()
        d_dst = torch.zeros(nrows, 32, dtype=torch.uint8, device="cuda")
        calls = lambda: (ccr_mod.ccr_alltoall_rows(c, s_d, r_d, counts, row),  # noqa: E731
                         ccr_mod.ccr_moe_topk(c, d_logits, d_topk),
                         ccr_mod.ccr_permute_rows(c, d_dst, d_src, d_idx))
        calls()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=torch.cuda.Stream()):
            calls()

        def reset():
            for t in r_d:
                t.zero_()
            d_topk.zero_()
            d_dst.zero_()

        def check(rep):
            for a, b in zip(r_d, ref):
                assert to_host(a)[:b.size].tobytes() == b.tobytes(), f"replay {rep}"
            np.testing.assert_array_equal(to_host(d_topk), ref_topk)
            np.testing.assert_array_equal(to_host(d_dst), src_rows[idx])

        _replays(torch, g, reset, check, calls)


def test_calls_that_cannot_replay_are_refused(ccr_mod):
    import torch
    R, n = 4, 4096
    xs = workloads.random_buffers(R, n, "bf16", seed=3, dist="normal", scale=1e-2)
    cases = [("sdma all-reduce", dict(copy_mode="sdma"),
              lambda c, b, m: ccr_mod.ccr_allreduce(c, b)),
             ("fp32-partials all-reduce", dict(bf16_acc="fp32_partials"),
              lambda c, b, m: ccr_mod.ccr_allreduce(c, b)),
             ("staged send/recv", dict(),
              lambda c, b, m: ccr_mod.ccr_sendrecv_batch(c, b[:2], b[2:])),
             ("sdma all-to-all", dict(copy_mode="sdma"),
              lambda c, b, m: ccr_mod.ccr_alltoall_rows(c, m[0], m[1], np.ones((R, R), np.int64), 16)),
             ("all-reduce with a CU budget", dict(cu_budget=64),
              lambda c, b, m: ccr_mod.ccr_allreduce(c, b)),
             ("all-to-all with a CU budget", dict(cu_budget=32),
              lambda c, b, m: ccr_mod.ccr_alltoall_rows(c, m[0], m[1], np.ones((R, R), np.int64), 16))]
    for name, cfg, call in cases:
        say(f"graph refusal: {name}")
        with ccr_mod.Context(0, ccr_mod.Config(**cfg)) as c:
            bufs = [to_dev(x) for x in xs]
            a2a = ([torch.zeros(R * 16, dtype=torch.uint8, device="cuda") for _ in range(R)],
                   [torch.zeros(R * 16, dtype=torch.uint8, device="cuda") for _ in range(R)])
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=torch.cuda.Stream()):
                with pytest.raises(ccr_mod.CcrError) as e:
                    call(c, bufs, a2a)
                bufs[0].add_(0)  # keep the captured graph non-empty
            assert e.value.status == ccr_mod.CCR_ERR_UNSUPPORTED, name
            assert "graph" in ccr_mod.ccr_last_error()
            call(c, bufs, a2a)  # the same call still runs eagerly
            torch.cuda.synchronize()


def test_captured_three_stage_moe_replays(ccr_mod):
    """Pack, exchange and unpack (kernel copies) and the combine, captured
    once from a plan made eagerly, replayed against the oracle."""
    import torch
    R, T, E, K, H = 4, 96, 16, 2, 64
    w = workloads.MOE_DISPATCH_BF16
    xs, logits = workloads.moe_inputs(w, tokens=T, R=R)
    xs = [x[:, :H].copy() for x in xs]
    logits = [l[:, :E].copy() for l in logits]
    ref = oracle.moe_dispatch(xs, [oracle.moe_topk(l, K) for l in logits], E)
    rows = [int(ref["counts"][:, d].sum()) for d in range(R)]
    say("graph three-stage moe")
    with ccr_mod.Context(0) as c:
        d_x = [to_dev(x) for x in xs]
        topk = [torch.zeros(T, K, dtype=torch.int32, device="cuda") for _ in range(R)]
        src_tok = [torch.zeros(T * K, dtype=torch.int32, device="cuda") for _ in range(R)]
        slot = [torch.zeros(T * K, dtype=torch.int32, device="cuda") for _ in range(R)]
        ecnt = []
        for r in range(R):
            ccr_mod.ccr_moe_topk(c, to_dev(logits[r]), topk[r])
            ecnt.append(ccr_mod.ccr_moe_plan(c, topk[r], E, R, src_tok[r], slot[r]))
        ecnt = np.stack(ecnt)
        send = [torch.zeros(T * K, H, dtype=torch.bfloat16, device="cuda") for _ in range(R)]
        recv = [torch.zeros(max(1, n), H, dtype=torch.bfloat16, device="cuda") for n in rows]
        exp = [torch.zeros(max(1, n), H, dtype=torch.bfloat16, device="cuda") for n in rows]
        out = [torch.zeros(T, K, H, dtype=torch.bfloat16, device="cuda") for _ in range(R)]
        calls = lambda: (ccr_mod.ccr_moe_dispatch(c, d_x, src_tok, ecnt, K, send, recv, exp),  # noqa: E731
                         ccr_mod.ccr_moe_combine(c, exp, slot, ecnt, T, K, recv, send, out))
        calls()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=torch.cuda.Stream()):
            calls()

        def reset():
            for t in send + recv + exp + out:
                t.zero_()

        def check(rep):
            for d in range(R):
                np.testing.assert_array_equal(to_host(exp[d])[:rows[d]], ref["exp"][d])
            for r in range(R):
                np.testing.assert_array_equal(to_host(out[r]), np.repeat(xs[r][:, None, :], K, axis=1))

        _replays(torch, g, reset, check, calls)


# ------------------------------------------------ the library's graph cache
_ORACLE = {"allreduce": lambda xs: oracle.ring_allreduce(xs, S=1),
           "reduce_scatter": lambda xs: oracle.ring_reduce_scatter(xs, S=1),
           "all_gather": lambda xs: oracle.ring_all_gather(xs, S=1)}


@pytest.mark.parametrize("which", ["allreduce", "reduce_scatter", "all_gather"])
@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_graph_cache_matches_eager(ccr_mod, dt, which):
    """Small ring calls repeated on the same buffers: the first runs eagerly,
    the second is captured, the rest replay; two buffer sets alternate; every
    call bit-exact against the oracle, before and after a configuration
    change (which drops the graphs) and with the cache off."""
    import torch
    # at least 12 hops, at most 2 MiB per rank: the calls the cache takes
    R, n = (8 if which == "allreduce" else 14), 3 * 65536 + 9
    xs = workloads.random_buffers(R, n, dt, seed=61, dist="normal", scale=1e-2)
    expect = _ORACLE[which](xs)
    fn = getattr(ccr_mod, f"ccr_{which}")
    say(f"graph cache {which} {dt}")
    with ccr_mod.Context(0) as c:
        src = [to_dev(x) for x in xs]
        sets = [[t.clone() for t in src] for _ in range(2)]

        def rounds(k):
            for call in range(k):
                for b in sets:
                    for t, x in zip(b, src):
                        t.copy_(x)
                for b in sets:
                    fn(c, b)
                torch.cuda.synchronize()
                for b in sets:
                    for q in range(R):
                        assert to_host(b[q]).tobytes() == expect[q].tobytes(), f"call {call} rank {q}"

        rounds(5)
        graphs, replays = ccr_mod.ccr_graph_cache_stats(c)
        assert graphs == 2 and replays == 2 * 4  # per set: eager, capture + replay, 3 replays
        c.set_config(ccr_mod.Config(slices=2))  # drops the graphs; still cached afterwards
        assert ccr_mod.ccr_graph_cache_stats(c) == (0, replays)
        rounds(3)
        assert ccr_mod.ccr_graph_cache_stats(c) == (2, replays + 2 * 2)
        c.set_config(ccr_mod.Config(graph_cache=False))
        rounds(2)
        assert ccr_mod.ccr_graph_cache_stats(c) == (0, replays + 2 * 2)


def test_graph_cache_replaces_least_recent(ccr_mod):
    """More buffer sets than the cache holds (32): each set is called twice
    in a row (eager, then captured and replayed), so every new set beyond
    the 32nd replaces a captured graph; every result exact."""
    import torch
    R, n, sets_n = 8, 4096 + 8, 36
    xs = workloads.random_buffers(R, n, "bf16", seed=62, dist="normal", scale=1e-2)
    expect = oracle.ring_allreduce(xs, S=1)
    say("graph cache eviction")
    with ccr_mod.Context(0) as c:
        src = [to_dev(x) for x in xs]
        sets = [[t.clone() for t in src] for _ in range(sets_n)]
        for rep in range(2):
            for i, b in enumerate(sets):
                for call in range(2):
                    for t, x in zip(b, src):
                        t.copy_(x)
                    ccr_mod.ccr_allreduce(c, b)
                    torch.cuda.synchronize()
                    for q in range(R):
                        assert to_host(b[q]).tobytes() == expect[q].tobytes(), \
                            f"rep {rep} set {i} call {call} rank {q}"
        graphs, replays = ccr_mod.ccr_graph_cache_stats(c)
        assert graphs == 32 and replays == 2 * sets_n
