"""The staged send/recv that allocates nothing (ccr_sendrecv_batch_noalloc),
called through the C ABI and checked byte for byte against the allocating
ccr_sendrecv_batch on the same inputs: two calls in a row, the second
smaller; the size limit of the fixed scratch; and a capture of the call
replayed with eager work between the replays."""
import numpy as np
import pytest

from gpu_helpers import raw_to_dev, say, to_host, torch_cuda

pytestmark = pytest.mark.gpu

SCRATCH_BYTES = 16 << 20


@pytest.fixture(scope="module")
def ccr_mod():
    torch_cuda()
    import collective_communication_reduce_amd as ccr
    return ccr


def _noalloc(ccr, ctx, send, recv, stream=None):
    """The C entry point itself (its ctypes signature comes from the binding)."""
    lib = ccr._lib
    nbytes = send[0].numel() * send[0].element_size()
    return lib.ccr_sendrecv_batch_noalloc(ctx.handle, ccr._ptrs(send), ccr._ptrs(recv), len(send),
                                          nbytes, ccr._stream(stream))


def _sources(n, nbytes, seed):
    rng = np.random.default_rng(seed)
    return [rng.integers(0, 256, nbytes, dtype=np.uint8) for _ in range(n)]


@pytest.mark.parametrize("chunk,slots", [(4 << 20, 2), (1 << 20, 3), (8 << 20, 2)])
def test_noalloc_matches_the_allocating_call_twice(ccr_mod, chunk, slots):
    import torch
    cfg = ccr_mod.Config(staging_chunk_bytes=chunk, staging_slots=slots)
    with ccr_mod.Context(0, cfg) as c:
        for m, nbytes, seed in ((4, 16 << 20, 1), (3, 5 * (1 << 20) + 4096 + 48, 2)):
            say(f"noalloc sendrecv chunk={chunk} slots={slots} m={m} nbytes={nbytes}")
            src = [raw_to_dev(x) for x in _sources(m, nbytes, seed)]
            want = [torch.zeros_like(x) for x in src]
            got = [torch.full_like(x, 7) for x in src]
            ccr_mod.ccr_sendrecv_batch(c, src, want)
            assert _noalloc(ccr_mod, c, src, got) == ccr_mod.CCR_OK, ccr_mod.ccr_last_error()
            torch.cuda.synchronize()
            for a, b, x in zip(got, want, src):
                assert to_host(a).tobytes() == to_host(b).tobytes() == to_host(x).tobytes()


def test_noalloc_rejects_what_it_cannot_stage(ccr_mod):
    import torch
    x = torch.arange(4096, dtype=torch.int32, device="cuda")
    y = torch.zeros_like(x)
    say("noalloc limits")
    with ccr_mod.Context(0, ccr_mod.Config(staging_chunk_bytes=SCRATCH_BYTES, staging_slots=2)) as c:
        assert _noalloc(ccr_mod, c, [x], [y]) == ccr_mod.CCR_ERR_INVALID_ARG
        assert "exceeds" in ccr_mod.ccr_last_error()
    with ccr_mod.Context(0, ccr_mod.Config(copy_mode="sdma")) as c:
        assert _noalloc(ccr_mod, c, [x], [y]) == ccr_mod.CCR_ERR_UNSUPPORTED
    torch.cuda.synchronize()
    assert not y.any()
    with ccr_mod.Context(0, ccr_mod.Config(staging_chunk_bytes=SCRATCH_BYTES // 2, staging_slots=2)) as c:
        assert _noalloc(ccr_mod, c, [x], [y]) == ccr_mod.CCR_OK
        torch.cuda.synchronize()
    assert torch.equal(x, y)


def test_noalloc_replays_from_a_graph(ccr_mod):
    """Captured on a side stream and replayed three times, each replay after
    eager work that overwrites the destinations and changes the sources."""
    import torch
    m, nbytes = 2, 3 << 20
    with ccr_mod.Context(0, ccr_mod.Config(staging_chunk_bytes=1 << 20, staging_slots=2)) as c:
        src = [raw_to_dev(x) for x in _sources(m, nbytes, 5)]
        dst = [torch.zeros_like(x) for x in src]
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):  # warm-up outside the capture
            assert _noalloc(ccr_mod, c, src, dst, s) == ccr_mod.CCR_OK
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            st = _noalloc(ccr_mod, c, src, dst, s)
        assert st == ccr_mod.CCR_OK, ccr_mod.ccr_last_error()
        for rep in range(3):
            say(f"noalloc graph replay {rep}")
            for x in src:
                x.add_(1)  # new contents, same buffers
            for d in dst:
                d.fill_(0)
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            for a, x in zip(dst, src):
                assert to_host(a).tobytes() == to_host(x).tobytes(), f"replay {rep}"


def _random_cases(seed=3131, n=40):
    """(case, chunk, slots, [(transfers, bytes)] x 2, the second call smaller),
    chunk x slots within the fixed scratch, at most ~2000 chunks per call."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        slots = int(rng.integers(1, 5))
        calls = sorted(((int(rng.integers(1, 6)), 16 * int(10 ** rng.uniform(0, 5.5))) for _ in range(2)),
                       key=lambda c: -c[0] * c[1])
        top = (SCRATCH_BYTES // slots) // 16
        low = -(-calls[0][0] * calls[0][1] // (2000 * 16))
        chunk = 16 * int(min(top, max(low, 10 ** rng.uniform(0, np.log10(top)))))
        out.append((i, chunk, slots, calls))
    return out


@pytest.mark.parametrize("case", _random_cases(), ids=lambda c: f"case{c[0]}")
def test_noalloc_random_shapes(ccr_mod, case):
    """Random chunk sizes, slot counts and transfers: two calls in a row (the
    second smaller), each byte for byte as the allocating call."""
    import torch
    i, chunk, slots, calls = case
    with ccr_mod.Context(0, ccr_mod.Config(staging_chunk_bytes=chunk, staging_slots=slots)) as c:
        for k, (m, nbytes) in enumerate(calls):
            say(f"noalloc random case {i} call {k}: chunk={chunk} slots={slots} m={m} nbytes={nbytes}")
            src = [raw_to_dev(x) for x in _sources(m, nbytes, 100 * i + k)]
            want = [torch.zeros_like(x) for x in src]
            got = [torch.full_like(x, 7) for x in src]
            ccr_mod.ccr_sendrecv_batch(c, src, want)
            assert _noalloc(ccr_mod, c, src, got) == ccr_mod.CCR_OK, ccr_mod.ccr_last_error()
            torch.cuda.synchronize()
            for a, b, x in zip(got, want, src):
                assert to_host(a).tobytes() == to_host(b).tobytes() == to_host(x).tobytes()
