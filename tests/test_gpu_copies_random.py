"""Seeded random sweep of the copy paths, each case compared byte for byte
with the oracle: staged send/recv batches and the ring shift (chunk sizes,
slot counts, transfer counts and ragged sizes), the all-to-all in rows
(1-64 ranks, empty and skewed flows, row sizes of 16 B to 1 KiB) and in
elements (per-pair counts or uniform), with kernel or SDMA copies (engine
caps, striping, chunking, the flag-word hand-over).  SDMA cases keep the
number of staged chunks bounded, since every engine copy has a fixed cost of
microseconds.  The cases are fixed by the seed."""
import numpy as np
import pytest

import oracle
import workloads
from gpu_helpers import raw_to_dev, say, to_dev, to_host, torch_cuda

pytestmark = pytest.mark.gpu

N_CASES = 500


def _mode(rng):
    if rng.random() < 0.6:
        return {"copy_mode": "kernel"}
    cfg = {"copy_mode": "sdma"}
    if rng.random() < 0.4:
        cfg["dma_engines"] = int(rng.integers(1, 5))
    if rng.random() < 0.3:
        cfg["dma_stripe"] = int(rng.integers(1, 4))
    if rng.random() < 0.3:
        cfg["dma_chunk_bytes"] = 16 * int(rng.integers(256, 8192))
    if rng.random() < 0.1:
        cfg["dma_sync"] = "stream_flags"
    return cfg


def _staging(rng, total_bytes, sdma):
    """A chunk size (multiple of 16) and slot count; SDMA: at most ~200 chunks."""
    slots = int(rng.integers(1, 6))
    chunk = 16 * int(10 ** rng.uniform(0, 4.3))
    if sdma:
        chunk = max(chunk, 16 * -(-total_bytes // (200 * 16)))
    return chunk, slots


def _cases(seed=77031):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(N_CASES):
        kind = str(rng.choice(["batch", "shift", "rows", "rows", "elements"]))
        cfg = _mode(rng)
        sdma = cfg["copy_mode"] == "sdma"
        if kind == "batch":
            m = int(rng.integers(1, 7))
            nbytes = 16 * int(10 ** rng.uniform(0, 4.8))
            chunk, slots = _staging(rng, m * nbytes, sdma)
            out.append((i, kind, cfg, dict(m=m, nbytes=nbytes, chunk=chunk, slots=slots)))
        elif kind == "shift":
            R = int(rng.integers(1, 17))
            dt = "bf16" if rng.random() < 0.5 else "f32"
            V = 8 if dt == "bf16" else 4
            count = V * int(10 ** rng.uniform(0, 4.5))
            chunk, slots = _staging(rng, R * count * 16 // V, sdma)
            out.append((i, kind, cfg, dict(R=R, dt=dt, count=count, chunk=chunk, slots=slots)))
        elif kind == "rows":
            # SDMA: fewer, smaller flows (each flow is one engine copy or more)
            R = int(rng.choice([1, 2, 3, 4, 5, 8, 12, 16] + ([] if sdma else [32, 64])))
            row_bytes = 16 * int(rng.integers(1, 65))
            cmax = int(rng.choice([1, 3, 10] + ([] if sdma else [100])))
            counts = rng.integers(0, cmax + 1, (R, R))
            counts[rng.random((R, R)) < 0.3] = 0
            if rng.random() < 0.2:
                counts[rng.integers(0, R), rng.integers(0, R)] = int(rng.integers(1000, 5000 if sdma else 20000))
            out.append((i, kind, cfg, dict(R=R, row_bytes=row_bytes, counts=counts)))
        else:
            R = int(rng.choice([1, 2, 3, 5, 8, 16, 32]))
            dt = "bf16" if rng.random() < 0.5 else "f32"
            V = 8 if dt == "bf16" else 4
            K = int(rng.integers(1, 200)) * R
            if rng.random() < 0.4:
                counts = None
                count = K * V
            else:
                counts = np.stack([rng.multinomial(K, rng.dirichlet(np.ones(R))) for _ in range(R)]) * V
                count = K * V
            out.append((i, kind, cfg, dict(R=R, dt=dt, count=count, counts=counts)))
    return out


CASES = _cases()


@pytest.fixture(scope="module")
def ccr_mod():
    torch_cuda()
    import collective_communication_reduce_amd as ccr
    return ccr


def _same(got: np.ndarray, want: np.ndarray, what: str):
    if got.tobytes() != want.tobytes():
        g, w = got.view(np.uint8), want.view(np.uint8)
        bad = np.nonzero(g != w)[0] if g.size == w.size else np.array([-1])
        raise AssertionError(f"{what}: {bad.size} bytes differ, first {bad[:5]}")


@pytest.mark.parametrize("case", CASES, ids=[f"case{c[0]}-{c[1]}" for c in CASES])
def test_random_copy_case(ccr_mod, case):
    import torch
    i, kind, cfg, p = case
    say(f"random copy case {i}: {kind} {cfg} " + " ".join(f"{k}={v}" for k, v in p.items() if k != "counts"))
    rng = np.random.default_rng(5000 + i)
    if kind == "batch":
        srcs = [rng.integers(0, 256, p["nbytes"], dtype=np.uint8) for _ in range(p["m"])]
        want, _ = oracle.staged_copy(srcs, p["chunk"], p["slots"])
        with ccr_mod.Context(0, ccr_mod.Config(staging_chunk_bytes=p["chunk"], staging_slots=p["slots"],
                                               **cfg)) as c:
            s = [raw_to_dev(x) for x in srcs]
            r = [torch.zeros_like(x) for x in s]
            ccr_mod.ccr_sendrecv_batch(c, s, r)
            torch.cuda.synchronize()
            for m in range(p["m"]):
                _same(to_host(r[m]), want[m], f"case {i} transfer {m}")
    elif kind == "shift":
        xs = workloads.random_buffers(p["R"], p["count"], p["dt"], seed=5000 + i, dist="normal")
        want, _ = oracle.ring_sendrecv([x.view(np.uint8) for x in xs], p["chunk"], p["slots"])
        with ccr_mod.Context(0, ccr_mod.Config(staging_chunk_bytes=p["chunk"], staging_slots=p["slots"],
                                               **cfg)) as c:
            s = [to_dev(x) for x in xs]
            r = [torch.zeros_like(x) for x in s]
            ccr_mod.ccr_sendrecv(c, s, r)
            torch.cuda.synchronize()
            for q in range(p["R"]):
                _same(to_host(r[q]).view(np.uint8), want[q], f"case {i} rank {q}")
    elif kind == "rows":
        R, row_bytes, counts = p["R"], p["row_bytes"], p["counts"]
        sends = [rng.integers(0, 256, int(counts[r].sum()) * row_bytes, dtype=np.uint8) for r in range(R)]
        want = oracle.alltoall(sends, counts, row_bytes)
        with ccr_mod.Context(0, ccr_mod.Config(**cfg)) as c:
            s = [raw_to_dev(x) if x.size else torch.zeros(16, dtype=torch.uint8, device="cuda") for x in sends]
            r = [torch.zeros(max(16, x.size), dtype=torch.uint8, device="cuda") for x in want]
            ccr_mod.ccr_alltoall_rows(c, s, r, counts, row_bytes)
            torch.cuda.synchronize()
            for d in range(R):
                _same(to_host(r[d])[:want[d].size], want[d], f"case {i} rank {d}")
    else:
        R, dt, count, counts = p["R"], p["dt"], p["count"], p["counts"]
        esize = 2 if dt == "bf16" else 4
        xs = workloads.random_buffers(R, count, dt, seed=5000 + i, dist="normal")
        full = counts if counts is not None else np.full((R, R), count // R, np.int64)
        want = oracle.alltoall([x.view(np.uint8) for x in xs], full, esize)
        tdt = torch.bfloat16 if dt == "bf16" else torch.float32
        with ccr_mod.Context(0, ccr_mod.Config(**cfg)) as c:
            s = [to_dev(x) for x in xs]
            r = [torch.zeros(max(1, int(full[:, d].sum())), dtype=tdt, device="cuda") for d in range(R)]
            ccr_mod.ccr_alltoall(c, s, r, counts)
            torch.cuda.synchronize()
            for d in range(R):
                got = to_host(r[d]).view(np.uint8)[:want[d].size]
                _same(got, want[d], f"case {i} rank {d}")
