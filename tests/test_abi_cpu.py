"""Host-side checks of the C-ABI library: it loads without a GPU, exports
every entry point the header declares, validates its configuration, and its
ring scheduler emits the textbook ring (checked against the oracle's
partition and against the ring's structural properties).  No GPU is used."""
import ctypes
import os
import re

import numpy as np
import pytest

import collective_communication_reduce_amd as ccr
import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _header_functions():
    text = open(os.path.join(ROOT, "include", "ccr.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return set(re.findall(r"\b(ccr_[a-z0-9_]+)\s*\(", text))


def test_library_exports_every_declared_symbol():
    names = _header_functions()
    assert len(names) >= 19
    lib = ctypes.CDLL(ccr.LIB_PATH)
    for n in sorted(names):
        assert hasattr(lib, n), f"libccr.so does not export {n}"
    assert names == set(ccr._SIGNATURES), "binding and header disagree"
    assert "gfx950" in ccr.ccr_version()


def test_config_defaults_and_environment(monkeypatch):
    for k in ("CCR_COPY_MODE", "CCR_CU_BUDGET", "CCR_SLICES", "CCR_OVERLAP",
              "CCR_STAGING_CHUNK", "CCR_STAGING_SLOTS", "CCR_BF16_ACC", "CCR_DMA_STRIPE",
              "CCR_DMA_CHUNK", "CCR_DMA_SYNC", "CCR_DMA_ENGINES", "CCR_GRAPH_CACHE",
              "CCR_DMA_DEADLINE_US"):
        monkeypatch.delenv(k, raising=False)
    c = ccr.ccr_config_default()
    assert c == ccr.Config("kernel", 0, 1, False, 4 << 20, 2, "per_hop", 0, 0, "host_func", 0, True, 0)
    monkeypatch.setenv("CCR_COPY_MODE", "sdma")
    monkeypatch.setenv("CCR_CU_BUDGET", "32")
    monkeypatch.setenv("CCR_SLICES", "4")
    monkeypatch.setenv("CCR_OVERLAP", "1")
    monkeypatch.setenv("CCR_STAGING_CHUNK", str(1 << 20))
    monkeypatch.setenv("CCR_STAGING_SLOTS", "3")
    monkeypatch.setenv("CCR_BF16_ACC", "fp32_partials")
    monkeypatch.setenv("CCR_DMA_STRIPE", "4")
    monkeypatch.setenv("CCR_DMA_CHUNK", str(1 << 21))
    monkeypatch.setenv("CCR_DMA_SYNC", "stream_flags")
    monkeypatch.setenv("CCR_DMA_ENGINES", "4")
    monkeypatch.setenv("CCR_GRAPH_CACHE", "0")
    monkeypatch.setenv("CCR_DMA_DEADLINE_US", "2500")
    assert ccr.ccr_config_default() == ccr.Config("sdma", 32, 4, True, 1 << 20, 3, "fp32_partials", 4,
                                                  1 << 21, "stream_flags", 4, False, 2500)
    monkeypatch.setenv("CCR_DMA_DEADLINE_US", "-1")
    with pytest.raises(ccr.CcrError):
        ccr.ccr_config_default()
    assert "dma_deadline_us" in ccr.ccr_last_error()
    monkeypatch.setenv("CCR_DMA_DEADLINE_US", "0")
    monkeypatch.setenv("CCR_GRAPH_CACHE", "2")
    with pytest.raises(ccr.CcrError):
        ccr.ccr_config_default()
    monkeypatch.setenv("CCR_GRAPH_CACHE", "1")
    monkeypatch.setenv("CCR_DMA_ENGINES", "17")
    with pytest.raises(ccr.CcrError) as e:
        ccr.ccr_config_default()
    assert "dma_engines" in ccr.ccr_last_error()
    monkeypatch.setenv("CCR_DMA_ENGINES", "0")
    monkeypatch.setenv("CCR_SLICES", "0")
    with pytest.raises(ccr.CcrError) as e:
        ccr.ccr_config_default()
    assert e.value.status == ccr.CCR_ERR_INVALID_ARG and "slices" in ccr.ccr_last_error()
    monkeypatch.setenv("CCR_SLICES", "2")
    monkeypatch.setenv("CCR_STAGING_CHUNK", "100")
    with pytest.raises(ccr.CcrError):
        ccr.ccr_config_default()


@pytest.mark.parametrize("R,count,S,dtype", [(1, 10, 1, 0), (2, 40, 1, 0), (3, 12, 1, 0),
                                             (4, 1 << 20, 2, 0), (5, 1001, 3, 1), (8, 26214400, 4, 1),
                                             (7, 3, 2, 0), (32, 8388608, 4, 0), (64, 1000, 2, 1),
                                             (6, 0, 1, 0)] + [
    # and 40 seeded random shapes
    (int(R), int(10 ** rng.uniform(0, 7)), int(rng.integers(1, 7)), int(rng.integers(0, 2)))
    for rng in [np.random.default_rng(5150)] for R in rng.integers(1, 34, 40)])
def test_ring_schedule_is_the_textbook_ring(R, count, S, dtype):
    V = 4 if dtype == 0 else 8
    ops = ccr.ccr_ring_schedule(R, count, S, dtype, which=0)
    assert len(ops) == 2 * R * (R - 1) * S
    # slice-major: all reduce-scatter hops of a slice, then its all-gather hops
    i = 0
    for s in range(S):
        for phase in (0, 1):
            for k in range(R - 1):
                hop = ops[i:i + R]
                i += R
                assert np.all(hop["slice"] == s) and np.all(hop["phase"] == phase)
                assert np.all(hop["step"] == k)
                # a perfect matching: every rank receives once and sends once, to q+1
                assert sorted(hop["dst_rank"].tolist()) == list(range(R))
                assert np.all(hop["src_rank"] == (hop["dst_rank"] - 1) % R)
                off = 2 if phase == 0 else 1
                assert np.all(hop["chunk"] == (hop["dst_rank"] - k - off) % R)
                # no (rank, chunk) is both written and read within a hop
                written = {(int(o["dst_rank"]), int(o["chunk"])) for o in hop}
                read = {(int(o["src_rank"]), int(o["chunk"])) for o in hop}
                assert not (written & read)
                for o in hop:
                    clo, chi = oracle.chunk_bounds(count, R, V, int(o["chunk"]))
                    assert (o["lo"], o["hi"]) == oracle.slice_bounds(clo, chi, S, V, s)
    # completeness: chunk c is reduced on ranks c+2, ..., c (the partial
    # travels c+1 -> c+2 -> ... -> c) and copied to every rank but c
    for s in range(S):
        for c in range(R):
            rs = ops[(ops["phase"] == 0) & (ops["slice"] == s) & (ops["chunk"] == c)]
            assert rs["dst_rank"].tolist() == [(c + 2 + k) % R for k in range(R - 1)]
            ag = ops[(ops["phase"] == 1) & (ops["slice"] == s) & (ops["chunk"] == c)]
            assert ag["dst_rank"].tolist() == [(c + 1 + k) % R for k in range(R - 1)]
    only_rs = ccr.ccr_ring_schedule(R, count, S, dtype, which=1)
    only_ag = ccr.ccr_ring_schedule(R, count, S, dtype, which=2)
    assert np.all(only_rs["phase"] == 0) and np.all(only_ag["phase"] == 1)
    assert len(only_rs) == len(only_ag) == R * (R - 1) * S


def test_ring_schedule_rejects_bad_arguments():
    for args in [(0, 10, 1, 0), (65, 10, 1, 0), (4, -1, 1, 0), (4, 10, 0, 0), (4, 10, 1, 7)]:
        with pytest.raises(ccr.CcrError) as e:
            ccr.ccr_ring_schedule(*args)
        assert e.value.status == ccr.CCR_ERR_INVALID_ARG


def test_null_arguments_are_rejected_without_a_device():
    lib = ccr._lib
    assert lib.ccr_allreduce(None, None, 4, 10, 0, None) == ccr.CCR_ERR_INVALID_ARG
    assert "ctx" in ccr.ccr_last_error()
    assert lib.ccr_ctx_create(0, None, None) == ccr.CCR_ERR_INVALID_ARG
    assert lib.ccr_ctx_destroy(None) == ccr.CCR_OK
    assert lib.ccr_config_default(None) == ccr.CCR_ERR_INVALID_ARG


@pytest.mark.parametrize("nbytes,deadline_us,gbs,max_e", [
    (314_572_800, 2950, 60.0, 14), (314_572_800, 1, 60.0, 14), (314_572_800, 10**7, 60.0, 14),
    (1, 1, 60.0, 3), (268_435_456, 700, 55.5, 4), (60_000, 1, 60.0, 16), (60_001, 1, 60.0, 16),
    (120_000, 1, 60.0, 16), (10**12, 1000, 0.5, 16)])
def test_dma_pace_is_the_fewest_engines_that_meet_the_deadline(nbytes, deadline_us, gbs, max_e):
    """The pick equals a brute-force search: the smallest E in 1..max_e with
    E engines x gbs x deadline >= bytes (exact integer arithmetic on the
    per-engine byte budget), else max_e."""
    got = ccr.ccr_dma_pace(nbytes, deadline_us, gbs, max_e)
    per_engine = deadline_us * 1e-6 * gbs * 1e9
    want = next((e for e in range(1, max_e + 1) if e * per_engine >= nbytes), max_e)
    assert got == want
    # no deadline, no rate, nothing to move, or no engines: nothing to pace
    assert ccr.ccr_dma_pace(nbytes, 0, gbs, max_e) == max_e
    assert ccr.ccr_dma_pace(nbytes, deadline_us, 0.0, max_e) == max_e
    assert ccr.ccr_dma_pace(0, deadline_us, gbs, max_e) == max_e
    assert ccr.ccr_dma_pace(nbytes, deadline_us, gbs, 0) == 0


TILE_BYTES = 2 * 256 * 16  # a ring-hop workgroup's tile: 2 x 256 16-byte vectors


@pytest.mark.parametrize("R,count,S,dtype", [
    (2, 1, 1, 0), (2, 1000, 3, 1), (3, 8, 1, 0), (3, 1001, 2, 0), (4, 4096 * 3 + 5, 1, 0),
    (5, 5 * 8192, 5, 1), (7, 3, 2, 1), (8, 26214400, 1, 1), (16, 4099, 5, 0), (17, 100003, 1, 1),
    (32, 8 * 1048576, 1, 0), (33, 70001, 2, 1), (64, 131077, 5, 0), (64, 2049, 1, 1),
    (4, 64, 5, 1), (6, 3 * 65536 + 11, 4, 0),
    # whole chunks of 48 bf16 and a ragged one of 40, 5 slices: slices 3 and 4
    # of a whole chunk are empty while slice 3 of the ragged chunk is not
    (2, 88, 5, 1)] + [
    # and 60 seeded random shapes
    (int(R), int(10 ** rng.uniform(0, 5.3 if R < 32 else 4.7)), int(rng.integers(1, 9)), int(rng.integers(0, 2)))
    for rng in [np.random.default_rng(8080)] for R in rng.choice([2, 3, 4, 5, 6, 7, 8, 9, 12, 16, 17, 31, 32, 64], 60)])
def test_ring_hop_layout_covers_the_schedule(R, count, S, dtype):
    """The ring-hop kernel's own index arithmetic (the function the kernel
    runs, called on the host): for every hop, its workgroups cover exactly
    the pieces the ring schedule lists for that hop -- every byte of every
    piece once, each piece's tiles contiguous and in order, the full chunks
    in destination-rank order (the ragged chunk last), so a hop starts on
    the chunk the previous hop wrote last."""
    esize = 4 if dtype == 0 else 2
    ops = ccr.ccr_ring_schedule(R, count, S, dtype, which=0)
    for s in range(S):
        for phase in (0, 1):
            for k in range(R - 1):
                hop = ops[(ops["slice"] == s) & (ops["phase"] == phase) & (ops["step"] == k)]
                want = sorted((int(o["src_rank"]), int(o["dst_rank"]), int(o["lo"]) * esize,
                               int(o["hi"] - o["lo"]) * esize) for o in hop if o["hi"] > o["lo"])
                rows = ccr.ccr_ring_hop_layout(R, count, S, dtype, phase, k, s)
                pieces = [tuple(int(x) for x in r[:4]) for r in rows]
                # runs of one piece each, tiles 0, 1, ... in workgroup order
                runs = []
                for i, p in enumerate(pieces):
                    if not runs or runs[-1][0] != p:
                        runs.append((p, []))
                    runs[-1][1].append(int(rows[i, 4]))
                assert sorted(p for p, _ in runs) == want, (s, phase, k)
                for p, tiles in runs:
                    assert tiles == list(range(-(-p[3] // TILE_BYTES))), (p, tiles[:4])
                # whole chunks (c < count // L) before the ragged one, in
                # destination-rank order
                V = 16 // esize
                L = -(-(-(-count // R)) // V) * V
                chunk = [p[2] // (L * esize) for p, _ in runs]
                whole = [c for c in chunk if c < count // L]
                assert chunk[:len(whole)] == whole and len(chunk) <= len(whole) + 1
                if len(whole) == R:
                    assert [p[1] for p, _ in runs] == list(range(R)), [p[1] for p, _ in runs]


def test_ring_hop_layout_past_32_bit_offsets():
    """3 ranks of 2^31 + 12345 bf16: byte offsets past 4 GiB, the ragged end
    in the last chunk; vectorised over the ~525,000 workgroups of a hop."""
    R, count = 3, (1 << 31) + 12345
    for phase, k in ((0, 0), (0, 1), (1, 1)):
        rows = ccr.ccr_ring_hop_layout(R, count, 1, 1, phase, k, 0)
        ops = ccr.ccr_ring_schedule(R, count, 1, 1, which=0)
        hop = ops[(ops["phase"] == phase) & (ops["step"] == k)]
        want = sorted((int(o["src_rank"]), int(o["dst_rank"]), int(o["lo"]) * 2,
                       int(o["hi"] - o["lo"]) * 2) for o in hop)
        keys, first = np.unique(rows[:, :4], axis=0, return_index=True)
        assert sorted(tuple(int(x) for x in r) for r in keys) == want
        for key in keys:
            t = rows[np.all(rows[:, :4] == key, axis=1), 4]
            assert np.array_equal(t, np.arange(-(-int(key[3]) // TILE_BYTES)))


def test_ring_hop_layout_refuses_what_the_kernel_does_not_take():
    # a chunk stride past 2^31 16-byte vectors (32 GiB per chunk): the hop
    # runs from a piece table instead
    with pytest.raises(ccr.CcrError) as e:
        ccr.ccr_ring_hop_layout(2, 1 << 36, 1, 0, 0, 0)
    assert e.value.status == ccr.CCR_ERR_UNSUPPORTED
    # one workgroup per 8 KiB tile, and a dispatch counts at most 2^32 - 1
    # work-items (2^24 - 1 workgroups of 256): 8 chunks of 2^21 tiles plus one
    # tile each are refused, 8 chunks of 2^21 - 1 tiles are taken
    with pytest.raises(ccr.CcrError) as e:
        ccr.ccr_ring_hop_layout(8, (1 << 35) + 64, 1, 0, 0, 0)
    assert e.value.status == ccr.CCR_ERR_UNSUPPORTED
    n = ctypes.c_int64()
    assert ccr._lib.ccr_ring_hop_layout(8, (1 << 35) - (1 << 14), 1, 0, 0, 0, 0, None, 0,
                                        ctypes.byref(n)) == ccr.CCR_OK
    assert n.value == 8 * ((1 << 21) - 1)
    for args in [(1, 10, 1, 0, 0, 0), (4, 10, 1, 0, 2, 0), (4, 10, 1, 0, 0, 3), (4, 10, 2, 0, 0, 0, 2),
                 (4, 10, 1, 5, 0, 0)]:
        with pytest.raises(ccr.CcrError) as e:
            ccr.ccr_ring_hop_layout(*args)
        assert e.value.status == ccr.CCR_ERR_INVALID_ARG


def test_config_names_are_checked_when_marshalled():
    """The binding maps the SDMA hand-over names to ccr_dma_sync_t values and
    refuses a name it does not know instead of sending a default."""
    for name, code in (("host_func", ccr.CCR_DMA_SYNC_HOST_FUNC), ("stream_flags", ccr.CCR_DMA_SYNC_STREAM_FLAGS)):
        c = ccr.Config(copy_mode="sdma", dma_sync=name).to_c()
        assert c.dma_sync == code and ccr.Config.from_c(c).dma_sync == name
    with pytest.raises(ValueError):
        ccr.Config(dma_sync="runtime").to_c()
