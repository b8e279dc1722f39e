"""GPU parity of the copy paths against the CPU oracle: staged P2P
send/recv, all-to-all and row permutes, in kernel and SDMA copy modes.
Copies are compared byte for byte."""
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


@pytest.mark.parametrize("mode", ["kernel", "sdma"])
@pytest.mark.parametrize("nbytes,chunk,slots,m", [(16, 4096, 2, 1), (4096 * 3 + 48, 4096, 2, 3),
                                                  (1 << 20, 1 << 18, 3, 2), (1 << 16, 1 << 16, 1, 2),
                                                  (4096, 4096, 4, 1), (5 * 4096 + 32, 4096, 4, 3),
                                                  (4096 + 16, 4096, 3, 5)])
def test_sendrecv_bytes(ccr_mod, mode, nbytes, chunk, slots, m):
    import torch
    rng = np.random.default_rng(nbytes + m)
    srcs = [rng.integers(0, 256, nbytes, dtype=np.uint8) for _ in range(m)]
    say(f"sendrecv {mode} nbytes={nbytes} chunk={chunk} slots={slots} m={m}")
    with ccr_mod.Context(0, ccr_mod.Config(copy_mode=mode, staging_chunk_bytes=chunk,
                                           staging_slots=slots)) as c:
        s = [raw_to_dev(x) for x in srcs]
        r = [torch.zeros_like(x) for x in s]
        ccr_mod.ccr_sendrecv_batch(c, s, r)
        torch.cuda.synchronize()
        dsts, _ = oracle.staged_copy(srcs, chunk, slots)
        for a, b in zip(r, dsts):
            assert to_host(a).tobytes() == b.tobytes()


@pytest.mark.parametrize("mode", ["kernel", "sdma"])
def test_sendrecv_full_pp_activations(ccr_mod, mode):
    """4 micro-batches of 2048 x 4096 bf16 through two 4 MiB slots."""
    import torch
    w = workloads.PP_STAGING_BF16
    mb = workloads.staging_inputs(w)
    say(f"sendrecv full {w.name} {mode}")
    with ccr_mod.Context(0, ccr_mod.Config(copy_mode=mode, staging_chunk_bytes=w.chunk_bytes,
                                           staging_slots=w.slots)) as c:
        s = [to_dev(x) for x in mb]
        r = [torch.empty_like(x) for x in s]
        ccr_mod.ccr_sendrecv_batch(c, s, r)
        torch.cuda.synchronize()
        for a, x in zip(r, mb):
            np.testing.assert_array_equal(to_host(a), x)


@pytest.mark.parametrize("mode", ["kernel", "sdma", "sdma-3-engines"])
@pytest.mark.parametrize("R,row_bytes", [(1, 16), (2, 48), (3, 4096), (8, 256), (20, 32)])
def test_alltoall_bytes(ccr_mod, mode, R, row_bytes):
    import torch
    rng = np.random.default_rng(R * row_bytes)
    counts = rng.integers(0, 9, (R, R))
    if R > 1:
        counts[1, 0] = 0
    sends = [rng.integers(0, 256, int(counts[r].sum()) * row_bytes, dtype=np.uint8) for r in range(R)]
    ref = oracle.alltoall(sends, counts, row_bytes)
    say(f"alltoall {mode} R={R} row_bytes={row_bytes}")
    cfg = ccr_mod.Config(copy_mode="sdma", dma_engines=3) if mode == "sdma-3-engines" else \
        ccr_mod.Config(copy_mode=mode)
    with ccr_mod.Context(0, cfg) as c:
        s = [raw_to_dev(x) if x.size else torch.zeros(16, dtype=torch.uint8, device="cuda") for x in sends]
        r = [torch.zeros(max(16, x.size), dtype=torch.uint8, device="cuda") for x in ref]
        ccr_mod.ccr_alltoall_rows(c, s, r, counts, row_bytes)
        torch.cuda.synchronize()
        for a, b in zip(r, ref):
            assert to_host(a)[:b.size].tobytes() == b.tobytes()


@pytest.mark.parametrize("nrows,nsrc,row_bytes", [(1, 1, 16), (1000, 333, 48), (24576, 4096, 4096),
                                                  (7, 100, 1040)])
def test_permute_rows_bytes(ccr_mod, nrows, nsrc, row_bytes):
    import torch
    rng = np.random.default_rng(nrows)
    src = rng.integers(0, 256, (nsrc, row_bytes), dtype=np.uint8)
    idx = rng.integers(0, nsrc, nrows).astype(np.int32)
    say(f"permute_rows nrows={nrows} nsrc={nsrc} row_bytes={row_bytes}")
    with ccr_mod.Context(0) as c:
        d_src = torch.from_numpy(src).cuda()
        d_dst = torch.zeros(nrows, row_bytes, dtype=torch.uint8, device="cuda")
        ccr_mod.ccr_permute_rows(c, d_dst, d_src, torch.from_numpy(idx).cuda())
        torch.cuda.synchronize()
        np.testing.assert_array_equal(to_host(d_dst), oracle.permute_rows(src, idx))


def test_permute_rows_skips_out_of_range_index(ccr_mod):
    import torch
    src = np.arange(4 * 16, dtype=np.uint8).reshape(4, 16)
    idx = np.array([3, -1, 4, 0], np.int32)
    say("permute_rows out-of-range entries")
    with ccr_mod.Context(0) as c:
        d_dst = torch.full((4, 16), 7, dtype=torch.uint8, device="cuda")
        ccr_mod.ccr_permute_rows(c, d_dst, torch.from_numpy(src).cuda(), torch.from_numpy(idx).cuda())
        torch.cuda.synchronize()
        out = to_host(d_dst)
    np.testing.assert_array_equal(out[0], src[3])
    np.testing.assert_array_equal(out[3], src[0])
    assert np.all(out[1] == 7) and np.all(out[2] == 7)


# ------------------------------------------------- SDMA engines + CPU proxy
def test_dma_engines_available(ccr_mod):
    say("dma engines")
    with ccr_mod.Context(0, ccr_mod.Config(copy_mode="sdma")) as c:
        ids = ccr_mod.ccr_dma_info(c)
    assert len(ids) >= 1 and len(set(ids)) == len(ids) and all(0 <= i < 16 for i in ids)


def test_dma_deadline_paces_every_sdma_call(ccr_mod):
    """With a deadline, each SDMA call is allowed ccr_dma_pace(its copy
    bytes, deadline, the measured engine rate, all engines) engines (a staged
    send/recv: at least that many, once one has completed), and the results
    stay those of the oracle, bit for bit."""
    import torch
    say("dma deadline pacing")
    R, n = 8, (1 << 18) + 40
    xs = workloads.random_buffers(R, n, "bf16", seed=91, dist="normal", scale=1.0)
    ref = oracle.ring_allreduce(xs, S=1)
    rng = np.random.default_rng(5)
    counts = rng.integers(0, 200, (R, R))
    row = 4096
    sends = [rng.integers(0, 256, int(counts[r].sum()) * row, dtype=np.uint8) for r in range(R)]
    a2a_ref = oracle.alltoall(sends, counts, row)
    mbs = [rng.integers(0, 256, 3 << 20, dtype=np.uint8) for _ in range(2)]
    with ccr_mod.Context(0, ccr_mod.Config(copy_mode="sdma")) as c:
        gbs, last = ccr_mod.ccr_dma_rate(c)
        assert last == 0 and 1.0 < gbs < 1000.0, gbs
        E = len(ccr_mod.ccr_dma_info(c))
        seen = set()
        first_staged = True
        for deadline in (1, 100, 2000, 10 ** 7, 0):
            c.set_config(ccr_mod.Config(copy_mode="sdma", dma_deadline_us=deadline))
            assert ccr_mod.ccr_dma_rate(c)[0] == gbs  # measured once, at proxy start
            # all-reduce: the all-gather's R-2 hops (the last reduce hop forwards)
            ts = [to_dev(x) for x in xs]
            ccr_mod.ccr_allreduce(c, ts)
            torch.cuda.synchronize()
            want = ccr_mod.ccr_dma_pace((R - 2) * n * 2, deadline, gbs, E)
            assert ccr_mod.ccr_dma_rate(c)[1] == want
            seen.add(want)
            for t, r in zip(ts, ref):
                assert to_host(t).tobytes() == r.tobytes()
            # all-to-all: every segment once
            sd = [raw_to_dev(x) for x in sends]
            rv = [torch.zeros(x.size, dtype=torch.uint8, device="cuda") for x in a2a_ref]
            ccr_mod.ccr_alltoall_rows(c, sd, rv, counts, row)
            torch.cuda.synchronize()
            assert ccr_mod.ccr_dma_rate(c)[1] == ccr_mod.ccr_dma_pace(int(counts.sum()) * row,
                                                                      deadline, gbs, E)
            for a, b in zip(rv, a2a_ref):
                assert to_host(a).tobytes() == b.tobytes()
            # staged send/recv: a fill and a drain per byte
            s = [raw_to_dev(x) for x in mbs]
            r = [torch.zeros_like(x) for x in s]
            ccr_mod.ccr_sendrecv_batch(c, s, r)
            torch.cuda.synchronize()
            # staged: ccr_dma_pace's count until a staged job has shown its cost per
            # chunk step, then the fewest engines whose modelled time fits -- never fewer
            used, floor = ccr_mod.ccr_dma_rate(c)[1], ccr_mod.ccr_dma_pace(2 * 2 * (3 << 20), deadline, gbs, E)
            assert (used == floor) if first_staged else (floor <= used <= E), (deadline, used, floor)
            first_staged = False
            for a, b in zip(r, mbs):
                assert to_host(a).tobytes() == b.tobytes()
        assert E in seen and (E == 1 or 1 in seen)  # both ends of the range were taken


@pytest.mark.parametrize("sync", ["host_func", "stream_flags"])
@pytest.mark.parametrize("m,nbytes,chunk,slots,stripe,engines",
                         [(4, 1 << 20, 1 << 18, 2, 0, 0), (3, 100000 // 16 * 16, 16384, 3, 2, 0),
                          (1, 4096, 4096, 1, 1, 0), (4, 1 << 20, 1 << 18, 2, 0, 2),
                          (2, 1 << 20, 1 << 17, 3, 3, 1)])
def test_sdma_staged_slot_state_machine(ccr_mod, m, nbytes, chunk, slots, stripe, engines, sync):
    """The proxy's staging slots follow idle -> filling -> draining -> idle,
    chunk i uses slot i mod slots, chunks fill in order, every chunk once,
    and the bytes arrive intact."""
    import torch
    rng = np.random.default_rng(nbytes)
    srcs = [rng.integers(0, 256, nbytes, dtype=np.uint8) for _ in range(m)]
    say(f"sdma staged m={m} nbytes={nbytes} chunk={chunk} slots={slots} stripe={stripe} "
        f"engines={engines} sync={sync}")
    with ccr_mod.Context(0, ccr_mod.Config(copy_mode="sdma", staging_chunk_bytes=chunk,
                                           staging_slots=slots, dma_stripe=stripe, dma_sync=sync,
                                           dma_engines=engines)) as c:
        s = [raw_to_dev(x) for x in srcs]
        r = [torch.zeros_like(x) for x in s]
        ccr_mod.ccr_sendrecv_batch(c, s, r)
        torch.cuda.synchronize()
        for a, b in zip(r, srcs):
            assert to_host(a).tobytes() == b.tobytes()
        log = ccr_mod.ccr_sendrecv_slot_log(c)
    nchunks = m * (-(-nbytes // chunk))
    assert len(log) == 3 * nchunks
    state = [0] * slots
    fills = []
    for ch, sl, st in log.tolist():
        assert sl == ch % slots
        assert (state[sl], st) in ((0, 1), (1, 2), (2, 0)), (state[sl], st)
        state[sl] = st
        if st == 1:
            fills.append(ch)
    assert fills == list(range(nchunks)) and state == [0] * slots


@pytest.mark.parametrize("sync", ["host_func", "stream_flags"])
def test_sdma_watchdog_reports_a_slow_operation(ccr_mod, sync):
    """With the proxy holding the release, a bounded wait on the stream
    times out; the stream is released afterwards and the result is exact."""
    import torch
    R, n = 4, 40000
    xs = workloads.random_buffers(R, n, "f32", seed=8, dist="normal")
    say(f"sdma watchdog sync={sync}")
    with ccr_mod.Context(0, ccr_mod.Config(copy_mode="sdma", dma_sync=sync)) as c:
        ts = [to_dev(x) for x in xs]
        torch.cuda.synchronize()
        ccr_mod.ccr_dma_hold_finish(c, 300_000)
        ccr_mod.ccr_allreduce(c, ts)
        assert ccr_mod.ccr_stream_wait(c, 30) == ccr_mod.CCR_ERR_TIMEOUT
        assert ccr_mod.ccr_stream_wait(c, 20_000) == ccr_mod.CCR_OK
        ccr_mod.ccr_dma_hold_finish(c, 0)
        ref = oracle.ring_allreduce(xs)
        for q, t in enumerate(ts):
            np.testing.assert_array_equal(to_host(t), ref[q])


@pytest.mark.parametrize("mode", ["kernel", "sdma"])
def test_sendrecv_edges(ccr_mod, mode):
    """Nothing to send; more transfers than slots; transfers smaller than one
    16-byte unit per striped engine; a ragged last chunk."""
    import torch
    say(f"sendrecv edges {mode}")
    with ccr_mod.Context(0, ccr_mod.Config(copy_mode=mode, staging_chunk_bytes=4096,
                                           staging_slots=2, dma_stripe=7)) as c:
        ccr_mod.ccr_sendrecv_batch(c, [], [])
        e = torch.zeros(0, dtype=torch.uint8, device="cuda")
        ccr_mod.ccr_sendrecv_batch(c, [e], [torch.zeros(0, dtype=torch.uint8, device="cuda")])
        for m, nbytes in ((9, 4096 * 2 + 16), (3, 48), (2, 16), (5, 4096 * 5 - 16)):
            rng = np.random.default_rng(m * 1000 + nbytes)
            srcs = [rng.integers(0, 256, nbytes, dtype=np.uint8) for _ in range(m)]
            s = [raw_to_dev(x) for x in srcs]
            r = [torch.zeros_like(x) for x in s]
            ccr_mod.ccr_sendrecv_batch(c, s, r)
            torch.cuda.synchronize()
            dsts, _ = oracle.staged_copy(srcs, 4096, 2)
            for a, b in zip(r, dsts):
                assert to_host(a).tobytes() == b.tobytes(), f"m={m} nbytes={nbytes}"


@pytest.mark.parametrize("mode,chunk", [("kernel", 0), ("sdma", 4096), ("sdma", 0)])
def test_alltoall_skewed_flows(ccr_mod, mode, chunk):
    """One flow of 10,000 rows among flows of 0-3 rows, cut into 4 KiB chunks
    on the SDMA engines (so the large flow spans many chunks and interleaves
    with the small ones) or with the automatic chunk size."""
    import torch
    R, row_bytes = 8, 64
    rng = np.random.default_rng(77)
    counts = rng.integers(0, 4, (R, R))
    counts[3, 5] = 10000
    sends = [rng.integers(0, 256, int(counts[r].sum()) * row_bytes, dtype=np.uint8) for r in range(R)]
    ref = oracle.alltoall(sends, counts, row_bytes)
    say(f"alltoall skewed {mode} chunk={chunk}")
    with ccr_mod.Context(0, ccr_mod.Config(copy_mode=mode, dma_chunk_bytes=chunk)) as c:
        s = [raw_to_dev(x) for x in sends]
        r = [torch.zeros(max(16, x.size), dtype=torch.uint8, device="cuda") for x in ref]
        ccr_mod.ccr_alltoall_rows(c, s, r, counts, row_bytes)
        torch.cuda.synchronize()
        for a, b in zip(r, ref):
            assert to_host(a)[:b.size].tobytes() == b.tobytes()


@pytest.mark.parametrize("mode", ["kernel", "sdma"])
def test_alltoall_max_ranks_and_empty(ccr_mod, mode):
    """64 ranks (4,096 flows, many of them empty), then an exchange with no
    rows at all."""
    import torch
    R, row_bytes = 64, 32
    rng = np.random.default_rng(64)
    counts = rng.integers(0, 3, (R, R))
    sends = [rng.integers(0, 256, int(counts[r].sum()) * row_bytes, dtype=np.uint8) for r in range(R)]
    ref = oracle.alltoall(sends, counts, row_bytes)
    say(f"alltoall R=64 {mode}")
    cfg = ccr_mod.Config(copy_mode="sdma", dma_engines=3) if mode == "sdma-3-engines" else \
        ccr_mod.Config(copy_mode=mode)
    with ccr_mod.Context(0, cfg) as c:
        s = [raw_to_dev(x) if x.size else torch.zeros(16, dtype=torch.uint8, device="cuda") for x in sends]
        r = [torch.zeros(max(16, x.size), dtype=torch.uint8, device="cuda") for x in ref]
        ccr_mod.ccr_alltoall_rows(c, s, r, counts, row_bytes)
        torch.cuda.synchronize()
        for a, b in zip(r, ref):
            assert to_host(a)[:b.size].tobytes() == b.tobytes()
        zero = np.zeros((R, R), np.int64)
        keep = [to_host(x) for x in r[:3]]
        ccr_mod.ccr_alltoall_rows(c, s, r, zero, row_bytes)
        torch.cuda.synchronize()
        for a, b in zip(r[:3], keep):
            assert to_host(a).tobytes() == b.tobytes()


def test_staging_allocation_failure_is_reported(ccr_mod):
    """A staging pool larger than the device holds: the call returns
    CCR_ERR_OOM and enqueues nothing, and the context works again once the
    configuration asks for a pool that fits."""
    import torch
    say("staging allocation failure")
    x = torch.arange(4096, dtype=torch.int32, device="cuda")
    y = torch.zeros_like(x)
    with ccr_mod.Context(0, ccr_mod.Config(staging_chunk_bytes=1 << 42, staging_slots=2)) as c:
        with pytest.raises(ccr_mod.CcrError) as e:
            ccr_mod.ccr_sendrecv_batch(c, [x], [y])
        assert e.value.status == ccr_mod.CCR_ERR_OOM, ccr_mod.ccr_last_error()
        torch.cuda.synchronize()
        assert not y.any()
        c.set_config(ccr_mod.Config())
        ccr_mod.ccr_sendrecv_batch(c, [x], [y])
        torch.cuda.synchronize()
        assert torch.equal(x, y)


# --------------------------------------------- the ring shift and element all-to-all
@pytest.mark.parametrize("mode", ["kernel", "sdma"])
@pytest.mark.parametrize("R,count,dt", [(1, 8, "f32"), (2, 4096 * 3 + 8, "bf16"), (5, 100000, "f32"),
                                        (8, 1 << 20, "bf16")])
def test_sendrecv_ring_shift(ccr_mod, mode, R, count, dt):
    """ccr_sendrecv: rank q receives rank q-1's buffer, through the staging
    slots (1 MiB chunks, 3 slots), byte for byte as the oracle's ring shift."""
    import torch
    xs = workloads.random_buffers(R, count, dt, seed=R * 101 + count, dist="normal")
    ref, _ = oracle.ring_sendrecv([x.view(np.uint8) for x in xs], 1 << 20, 3)
    say(f"sendrecv ring shift {mode} R={R} count={count} {dt}")
    with ccr_mod.Context(0, ccr_mod.Config(copy_mode=mode, staging_chunk_bytes=1 << 20,
                                           staging_slots=3)) as c:
        s = [to_dev(x) for x in xs]
        r = [torch.zeros_like(x) for x in s]
        ccr_mod.ccr_sendrecv(c, s, r)
        torch.cuda.synchronize()
        for q in range(R):
            assert to_host(r[q]).view(np.uint8).tobytes() == ref[q].tobytes(), f"rank {q}"


def test_sendrecv_ring_shift_rejects_bad_arguments(ccr_mod):
    import torch
    say("sendrecv ring shift: invalid arguments")
    a = [torch.zeros(1000, device="cuda") for _ in range(3)]
    b = [torch.zeros(1000, device="cuda") for _ in range(3)]
    with ccr_mod.Context(0) as c:
        lib = ccr_mod._lib
        with pytest.raises(ccr_mod.CcrError) as e:  # 999 fp32: not whole 16-byte vectors
            ccr_mod.ccr_sendrecv(c, [x[:999] for x in a], [x[:999] for x in b])
        assert e.value.status == ccr_mod.CCR_ERR_INVALID_ARG and "16-byte" in ccr_mod.ccr_last_error()
        with pytest.raises(ccr_mod.CcrError):  # a receive buffer that is also a send buffer
            ccr_mod.ccr_sendrecv(c, a, [b[0], a[2], b[2]])
        assert lib.ccr_sendrecv(c.handle, ccr_mod._ptrs(a), ccr_mod._ptrs(b), 0, 1000, 0, None) == \
            ccr_mod.CCR_ERR_INVALID_ARG
        assert lib.ccr_sendrecv(c.handle, ccr_mod._ptrs(a), ccr_mod._ptrs(b), 3, 1000, 7, None) == \
            ccr_mod.CCR_ERR_INVALID_ARG
        assert lib.ccr_sendrecv(c.handle, ccr_mod._ptrs(a), ccr_mod._ptrs(b), 3, 0, 0, None) == ccr_mod.CCR_OK


def _compositions(rng, R, K):
    """R rows of R non-negative integers, each row summing to K."""
    return np.stack([rng.multinomial(K, rng.dirichlet(np.ones(R))) for _ in range(R)])


@pytest.mark.parametrize("mode", ["kernel", "sdma"])
@pytest.mark.parametrize("R,dt,uniform", [(1, "f32", True), (3, "bf16", False), (8, "f32", True),
                                          (8, "bf16", False), (16, "f32", False), (64, "bf16", True)])
def test_alltoall_elements(ccr_mod, mode, R, dt, uniform):
    """ccr_alltoall over (count, dtype): counts in elements or NULL for
    count / R each; byte for byte as the oracle's all-to-all of one-element
    rows."""
    import torch
    V, esize = (4, 4) if dt == "f32" else (8, 2)
    rng = np.random.default_rng(R * 7 + (1 if uniform else 0))
    if uniform:
        count = R * V * 37
        counts = np.full((R, R), count // R, np.int64)
    else:
        K = 41 * R
        counts = _compositions(rng, R, K) * V
        count = K * V
        counts[R - 1, 0] = counts[R - 1, 0] + counts[R - 1, R - 1] if R > 1 else counts[0, 0]
        if R > 1:
            counts[R - 1, R - 1] = 0  # an empty segment
    xs = workloads.random_buffers(R, count, dt, seed=R, dist="normal")
    ref = oracle.alltoall([x.view(np.uint8) for x in xs], counts, esize)
    say(f"alltoall elements {mode} R={R} {dt} uniform={uniform}")
    with ccr_mod.Context(0, ccr_mod.Config(copy_mode=mode)) as c:
        s = [to_dev(x) for x in xs]
        tdt = torch.float32 if dt == "f32" else torch.bfloat16
        r = [torch.zeros(int(counts[:, d].sum()), dtype=tdt, device="cuda") for d in range(R)]
        ccr_mod.ccr_alltoall(c, s, r, None if uniform else counts)
        torch.cuda.synchronize()
        for d in range(R):
            assert to_host(r[d]).view(np.uint8).tobytes() == ref[d].tobytes(), f"rank {d}"
        if R > 1:  # a ragged segment and a row that does not sum to count are refused
            bad = counts.copy()
            bad[0, 0] += 1
            bad[0, 1] -= 1 if bad[0, 1] > 0 else 0
            with pytest.raises(ccr_mod.CcrError):
                ccr_mod.ccr_alltoall(c, s, r, bad)
            bad = counts.copy()
            bad[0, 0] += V
            with pytest.raises(ccr_mod.CcrError) as e:
                ccr_mod.ccr_alltoall(c, s, r, bad)
            assert "not count" in ccr_mod.ccr_last_error()


# ------------------------------------------------------- proxy shutdown
@pytest.mark.parametrize("sync", ["host_func", "stream_flags"])
def test_destroy_abandons_jobs_whose_stream_has_not_arrived(ccr_mod, monkeypatch, sync):
    """A context destroyed while its SDMA job still waits behind a GPU sleep
    on the caller's stream: after the (shortened) wait the job is abandoned,
    ccr_ctx_destroy reports it, and the stream, reaching the job later, goes
    on without it.  Every kernel here ends on its own (the sleep is bounded);
    the condition is forced from the host."""
    import time

    import torch
    R, n = 4, 40000
    xs = workloads.random_buffers(R, n, "f32", seed=12, dist="normal")
    say(f"destroy with a queued SDMA job, sync={sync}")
    # calibrate the GPU sleep: about one second
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    torch.cuda._sleep(10_000_000)
    e1.record()
    torch.cuda.synchronize()
    # (about 5 ms at the GPU's clock; the factor is bounded, so the sleep
    # lasts at most 400 times the calibration run)
    cycles = int(10_000_000 * min(400.0, 1000.0 / max(1e-3, e0.elapsed_time(e1))))
    s = torch.cuda.Stream()
    ts = [to_dev(x) for x in xs]
    c = ccr_mod.Context(0, ccr_mod.Config(copy_mode="sdma", dma_sync=sync))
    ccr_mod.ccr_allreduce(c, ts)  # starts the proxy
    torch.cuda.synchronize()
    monkeypatch.setenv("CCR_DESTROY_TIMEOUT_MS", "100")
    with torch.cuda.stream(s):
        torch.cuda._sleep(cycles)
        ccr_mod.ccr_allreduce(c, ts, stream=s)
    t0 = time.perf_counter()
    st = ccr_mod._lib.ccr_ctx_destroy(c.handle)
    c.handle = ctypes_null()
    dt = time.perf_counter() - t0
    assert st == ccr_mod.CCR_ERR_TIMEOUT and "abandoned" in ccr_mod.ccr_last_error(), ccr_mod.ccr_last_error()
    assert dt < 0.9, dt
    s.synchronize()  # the stream passes the abandoned job once the sleep ends
    monkeypatch.delenv("CCR_DESTROY_TIMEOUT_MS")
    with ccr_mod.Context(0, ccr_mod.Config(copy_mode="sdma", dma_sync=sync)) as c2:  # the GPU works on
        ts = [to_dev(x) for x in xs]
        ccr_mod.ccr_allreduce(c2, ts)
        torch.cuda.synchronize()
        ref = oracle.ring_allreduce(xs)
        for q, t in enumerate(ts):
            np.testing.assert_array_equal(to_host(t), ref[q])


def ctypes_null():
    import ctypes
    return ctypes.c_void_p()


@pytest.mark.parametrize("mode", ["kernel", "sdma"])
def test_ring_shift_and_element_alltoall_at_workload_sizes(ccr_mod, mode):
    """The boundary's two §8(b) forms at the workloads' sizes: the ring shift
    over R = 2 (a pipeline pair exchanging one 2048 x 4096 bf16 activation in
    each direction through two 4 MiB slots) and the uniform element
    all-to-all over 8 ranks of 4096 x 2048 bf16 (each rank's buffer cut into
    8 equal segments); both byte for byte against the oracle."""
    import torch
    w = workloads.PP_STAGING_BF16
    mb = workloads.staging_inputs(w)[:2]
    ref, _ = oracle.ring_sendrecv([x.view(np.uint8) for x in mb], w.chunk_bytes, w.slots)
    say(f"ring shift R=2 at {w.name} size, {mode}")
    with ccr_mod.Context(0, ccr_mod.Config(copy_mode=mode, staging_chunk_bytes=w.chunk_bytes,
                                           staging_slots=w.slots)) as c:
        s = [to_dev(x) for x in mb]
        r = [torch.zeros_like(x) for x in s]
        ccr_mod.ccr_sendrecv(c, s, r)
        torch.cuda.synchronize()
        for q in range(2):
            assert to_host(r[q]).view(np.uint8).tobytes() == ref[q].tobytes(), f"rank {q}"
    m = workloads.MOE_DISPATCH_BF16
    xs, _ = workloads.moe_inputs(m)
    count = m.tokens * m.hidden
    counts = np.full((m.R, m.R), count // m.R, np.int64)
    ref = oracle.alltoall([x.view(np.uint8) for x in xs], counts, 2)
    say(f"uniform element all-to-all at {m.name} size, {mode}")
    with ccr_mod.Context(0, ccr_mod.Config(copy_mode=mode)) as c:
        s = [to_dev(x.reshape(-1)) for x in xs]
        r = [torch.zeros_like(x) for x in s]
        ccr_mod.ccr_alltoall(c, s, r)
        torch.cuda.synchronize()
        for d in range(m.R):
            assert to_host(r[d]).view(np.uint8).tobytes() == ref[d].tobytes(), f"rank {d}"
