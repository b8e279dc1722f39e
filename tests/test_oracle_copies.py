"""Pins of the CPU oracle's copy paths: staged point-to-point transfer,
all-to-all and row permutation.  No GPU is needed."""
import os

import numpy as np
import pytest

import oracle
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_staged_copy_golden_slot_sequence():
    """Slot states of one 16 MiB transfer in 4 MiB chunks through 2 slots
    follow the hand-worked fixture (idle -> filling -> draining -> idle,
    chunk i in slot i mod 2)."""
    rows = [l.split("#")[0].split() for l in open(os.path.join(GOLDEN, "staging_4chunks_2slots.txt"))]
    expect = np.array([[int(v) for v in r] for r in rows if r], np.int32)
    src = np.random.default_rng(0).integers(0, 256, 16 << 20, dtype=np.uint8)
    dsts, ev = oracle.staged_copy([src], 4 << 20, 2)
    np.testing.assert_array_equal(ev, expect)
    assert dsts[0].tobytes() == src.tobytes()


@pytest.mark.parametrize("nbytes,chunk,slots,m", [(1, 4, 2, 1), (4099, 1024, 2, 3), (0, 16, 2, 2),
                                                  (1 << 16, 1 << 16, 1, 2), (12345, 1000, 3, 4)])
def test_staged_copy_moves_bytes_and_keeps_slot_discipline(nbytes, chunk, slots, m):
    rng = np.random.default_rng(nbytes)
    srcs = [rng.integers(0, 256, nbytes, dtype=np.uint8) for _ in range(m)]
    dsts, ev = oracle.staged_copy(srcs, chunk, slots)
    for s, d in zip(srcs, dsts):
        assert s.tobytes() == d.tobytes()
    nchunks = m * (-(-nbytes // chunk))
    assert len(ev) == 3 * nchunks
    state = [0] * slots
    seen = []
    for ch, sl, st in ev:
        assert sl == ch % slots
        assert st == (state[sl] + 1) % 3 if state[sl] != 2 else st == 0
        state[sl] = st
        if st == 1:
            seen.append(ch)
    assert seen == list(range(nchunks)) and state == [0] * slots


def _tagged_rows(R, counts, width):
    """Send buffers whose rows encode (source, destination, index)."""
    sends = []
    for r in range(R):
        rows = []
        for d in range(R):
            for j in range(counts[r][d]):
                rows.append(np.full(width, r * 1_000_000 + d * 10_000 + j, np.int32))
        sends.append(np.array(rows, np.int32).reshape(-1, width))
    return sends


@pytest.mark.parametrize("R", [1, 2, 3, 8])
def test_alltoall_layout_and_round_trip(R):
    """Receiver d holds, in source order, exactly the rows source r packed
    for d; the transposed exchange brings every row home."""
    rng = np.random.default_rng(R)
    counts = rng.integers(0, 6, (R, R))
    if R > 1:
        counts[0, 1] = 0  # an empty segment
    width = 3
    sends = _tagged_rows(R, counts, width)
    recvs = oracle.alltoall(sends, counts, width * 4)
    for d in range(R):
        got = recvs[d].view(np.int32).reshape(-1, width)
        expect = [r * 1_000_000 + d * 10_000 + j for r in range(R) for j in range(counts[r][d])]
        np.testing.assert_array_equal(got[:, 0], np.array(expect, np.int32))
        assert np.all(got == got[:, :1])
    back = oracle.alltoall([r.view(np.int32).reshape(-1, width) for r in recvs], counts.T, width * 4)
    for r in range(R):
        assert back[r].tobytes() == sends[r].tobytes()
    assert sum(x.size for x in recvs) == counts.sum() * width * 4


def test_permute_rows_is_numpy_take():
    rng = np.random.default_rng(9)
    src = rng.integers(0, 1 << 16, (301, 24), dtype=np.uint16)
    idx = rng.integers(0, 301, 517).astype(np.int32)
    np.testing.assert_array_equal(oracle.permute_rows(src, idx), np.take(src, idx, axis=0))
    assert oracle.permute_rows(src, np.zeros(0, np.int32)).shape == (0, 24)
    with pytest.raises(ValueError):
        oracle.permute_rows(src, np.array([301], np.int32))


def test_staging_workload_shape():
    w = workloads.PP_STAGING_BF16
    mb = workloads.staging_inputs(w, rows=8)
    assert len(mb) == 4 and mb[0].shape == (8, 4096) and mb[0].dtype == np.uint16
    assert w.rows * w.cols * 2 == 16 << 20 and w.chunk_bytes == 4 << 20


@pytest.mark.parametrize("R,nbytes,chunk,slots", [(1, 64, 16, 2), (2, 4096 * 3, 4096, 2),
                                                  (5, 1000, 96, 3), (8, 48, 4096, 2)])
def test_ring_sendrecv_shifts_each_rank_to_its_successor(R, nbytes, chunk, slots):
    """Rank q receives exactly what rank q-1 sent (tagged bytes name the
    sender), through the same slot discipline as the directed transfers:
    transfer r's chunks come r-th in the slot sequence."""
    sends = [np.full(nbytes, (r * 37 + 11) % 256, np.uint8) for r in range(R)]
    recvs, ev = oracle.ring_sendrecv(sends, chunk, slots)
    for q in range(R):
        assert recvs[q].tobytes() == bytes([((q - 1) % R * 37 + 11) % 256]) * nbytes
    per = -(-nbytes // chunk)
    fills = [int(ch) for ch, sl, st in ev if st == 1]
    assert fills == list(range(R * per))
    assert all(sl == ch % slots for ch, sl, _ in ev)
