"""CPU oracle for the ring all-reduce hot path -- TEST INFRASTRUCTURE ONLY.

Plain, slow, obviously-correct reference implementations that the GPU
library is checked against.  Only the test suite, the package smoke check
and the benchmark's ``cpu_baseline`` leg may import this package; the GPU
library never does, and this package never imports the GPU library.  The two
share no code: the arithmetic lives in ``ccr_oracle.c`` (plain C, built with
gcc, no fast-math, no FMA contraction) and in the short numpy compositions
below.

Source: "HOCCL: Offloading Collective Communication from GPU Cores to
Accelerate Distributed Training".  The paper scopes reductions out of its DMA
offload (§5 Limitations) and describes no ring; the ring reduce-scatter /
all-gather computed here is the textbook ring, built from per-hop
point-to-point transfers the way §3.4 (Collective Scheduler, Fig. 6) builds
collectives from P2P flows.  The readings where the paper is silent are
listed at the top of ``ccr_oracle.c``.

Every function here is pinned by ``tests/test_oracle_*.py`` against facts
that do not come from the oracle itself (brute-force sums of exactly
representable values, rounding-error bounds, a library bf16 conversion,
hand-worked fixtures under ``tests/golden/``, and invariants).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ccr_oracle.c")
_LIB = os.path.join(_HERE, "libccr_oracle.so")

F32, BF16, BF16_P32 = 0, 1, 2  # dtype codes of the C oracle


def build(force: bool = True) -> str:
    """Compile ccr_oracle.c into libccr_oracle.so with gcc."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call([
            "gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
            "-fno-fast-math", "-Wall", "-Werror", "-o", tmp, _SRC])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    """The loaded C oracle; built first if it is not there yet."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        L = ctypes.CDLL(_LIB)
        i64, i32, vp = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p
        P64 = ctypes.POINTER(ctypes.c_int64)
        L.orc_chunk_bounds.argtypes = [i64, i32, i32, i32, P64, P64]
        L.orc_slice_bounds.argtypes = [i64, i64, i32, i32, i32, P64, P64]
        L.orc_ring_reduce_scatter.argtypes = [vp, vp, i32, i64, i32, i32]
        L.orc_ring_all_gather.argtypes = [vp, i32, i64, i32, i32]
        L.orc_ring_allreduce.argtypes = [vp, vp, i32, i64, i32, i32]
        L.orc_ring_allreduce_range.argtypes = [vp, vp, i32, i64, i32, i32, i64, i64]
        L.orc_ring_step.argtypes = [vp, vp, i32, i64, i32, i32, i32, i32, i32]
        L.orc_fold.argtypes = [vp, i32, i64, i32, vp]
        L.orc_fold_at.argtypes = [vp, i32, i64, i32, vp, i64, vp]
        L.orc_f32_to_bf16.argtypes = [ctypes.c_float]
        L.orc_f32_to_bf16.restype = ctypes.c_uint16
        L.orc_bf16_to_f32.argtypes = [ctypes.c_uint16]
        L.orc_bf16_to_f32.restype = ctypes.c_float
        L.orc_f32_to_bf16_array.argtypes = [vp, vp, i64]
        L.orc_bf16_to_f32_array.argtypes = [vp, vp, i64]
        L.orc_staged_copy.argtypes = [vp, vp, i32, i64, i64, i32, vp, vp, i64]
        L.orc_staged_copy.restype = i64
        L.orc_alltoall.argtypes = [vp, vp, i32, vp, i64]
        L.orc_permute_rows.argtypes = [vp, vp, vp, i64, i64, i64]
        L.orc_moe_topk.argtypes = [vp, i64, i32, i32, vp]
        L.orc_moe_plan.argtypes = [vp, i64, i32, i32, i32, vp, vp, vp, vp]
        L.orc_moe_unpack_index.argtypes = [vp, i32, i32, i32, vp]
        _lib = L
    return _lib


def _ptrs(arrays):
    arr = (ctypes.c_void_p * len(arrays))(*[a.ctypes.data for a in arrays])
    return arr


def _check(rc):
    if rc != 0:
        raise ValueError(f"oracle rejected its arguments (code {rc})")


def _code(dtype, bf16_acc="per_hop"):
    if dtype == np.float32:
        return F32
    if dtype == np.uint16:
        return BF16 if bf16_acc == "per_hop" else BF16_P32
    raise TypeError("oracle buffers are float32, or uint16 holding bf16 bits")


# ----------------------------------------------------------------- partition
def chunk_bounds(n: int, R: int, vec: int, c: int):
    lo, hi = ctypes.c_int64(), ctypes.c_int64()
    lib().orc_chunk_bounds(n, R, vec, c, ctypes.byref(lo), ctypes.byref(hi))
    return lo.value, hi.value


def slice_bounds(clo: int, chi: int, S: int, vec: int, s: int):
    lo, hi = ctypes.c_int64(), ctypes.c_int64()
    lib().orc_slice_bounds(clo, chi, S, vec, s, ctypes.byref(lo), ctypes.byref(hi))
    return lo.value, hi.value


# --------------------------------------------------------------------- bf16
def f32_to_bf16(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, np.uint16)
    lib().orc_f32_to_bf16_array(x.ctypes.data, out.ctypes.data, x.size)
    return out


def bf16_to_f32(h: np.ndarray) -> np.ndarray:
    h = np.ascontiguousarray(h, dtype=np.uint16)
    out = np.empty(h.shape, np.float32)
    lib().orc_bf16_to_f32_array(h.ctypes.data, out.ctypes.data, h.size)
    return out


# --------------------------------------------------------------------- ring
def _prep(bufs):
    bufs = [np.ascontiguousarray(b) for b in bufs]
    n = bufs[0].size
    dt = bufs[0].dtype
    for b in bufs:
        if b.size != n or b.dtype != dt:
            raise ValueError("all ranks need the same element count and dtype")
    return bufs, n, dt


def ring_reduce_scatter(bufs, S: int = 1, bf16_acc: str = "per_hop"):
    """In place on copies; returns the R buffers after the ring reduce-scatter."""
    bufs, n, dt = _prep([b.copy() for b in bufs])
    code = _code(dt, bf16_acc)
    part = [np.zeros(n, np.float32) for _ in bufs] if code == BF16_P32 else []
    _check(lib().orc_ring_reduce_scatter(_ptrs(bufs), _ptrs(part) if part else None,
                                         len(bufs), n, S, code))
    return bufs


def ring_step(bufs, phase: str, k: int, s: int = 0, S: int = 1, part=None,
              bf16_acc: str = "per_hop"):
    """One hop, in place: phase "rs" (reduce-scatter step k) or "ag"."""
    bufs, n, dt = _prep(bufs)
    code = _code(dt, bf16_acc)
    _check(lib().orc_ring_step(_ptrs(bufs), _ptrs(part) if part else None, len(bufs), n, S,
                               s, k, 0 if phase == "rs" else 1, code))
    return bufs


def ring_all_gather(bufs, S: int = 1):
    bufs, n, dt = _prep([b.copy() for b in bufs])
    _check(lib().orc_ring_all_gather(_ptrs(bufs), len(bufs), n, S, dt.itemsize))
    return bufs


def ring_allreduce(bufs, S: int = 1, bf16_acc: str = "per_hop", inplace: bool = False):
    """Ring all-reduce (reduce-scatter then all-gather, slice-major)."""
    bufs = list(bufs) if inplace else [b.copy() for b in bufs]
    bufs, n, dt = _prep(bufs)
    code = _code(dt, bf16_acc)
    part = [np.zeros(n, np.float32) for _ in bufs] if code == BF16_P32 else []
    _check(lib().orc_ring_allreduce(_ptrs(bufs), _ptrs(part) if part else None,
                                    len(bufs), n, S, code))
    return bufs


def ring_allreduce_range(bufs, lo: int, hi: int, S: int = 1, bf16_acc: str = "per_hop",
                         part=None):
    """In place: the ring all-reduce of ``ring_allreduce`` on elements
    [lo, hi) of every buffer only (every hop, in the same order).  Element
    results depend on no other element, so disjoint ranges covering the
    buffers give exactly the unsplit result, in any order or at once."""
    bufs, n, dt = _prep(bufs)
    code = _code(dt, bf16_acc)
    if code == BF16_P32 and part is None:
        raise ValueError("fp32 partials need the R partial buffers")
    _check(lib().orc_ring_allreduce_range(_ptrs(bufs), _ptrs(part) if part else None, len(bufs),
                                          n, S, code, lo, hi))
    return bufs


def ring_allreduce_threads(bufs, threads: int, S: int = 1, bf16_acc: str = "per_hop"):
    """``ring_allreduce`` with the element range cut into ``threads`` equal
    parts, each run by ``ring_allreduce_range`` on a thread of its own (the C
    call releases Python's lock).  Returns new buffers."""
    from concurrent.futures import ThreadPoolExecutor
    bufs, n, dt = _prep([b.copy() for b in bufs])
    part = [np.zeros(n, np.float32) for _ in bufs] if _code(dt, bf16_acc) == BF16_P32 else None
    T = max(1, int(threads))
    cuts = [n * t // T for t in range(T + 1)]
    with ThreadPoolExecutor(T) as ex:
        list(ex.map(lambda t: ring_allreduce_range(bufs, cuts[t], cuts[t + 1], S, bf16_acc, part),
                    range(T)))
    return bufs


def fold(xs, bf16_acc: str = "per_hop"):
    """Closed form of the ring result (one buffer, identical on every rank)."""
    xs, n, dt = _prep(xs)
    out = np.empty(n, dt)
    _check(lib().orc_fold(_ptrs(xs), len(xs), n, _code(dt, bf16_acc), out.ctypes.data))
    return out


def fold_at(xs, idx, bf16_acc: str = "per_hop"):
    xs, n, dt = _prep(xs)
    idx = np.ascontiguousarray(idx, dtype=np.int64)
    out = np.empty(idx.size, dt)
    _check(lib().orc_fold_at(_ptrs(xs), len(xs), n, _code(dt, bf16_acc),
                             idx.ctypes.data, idx.size, out.ctypes.data))
    return out


# ------------------------------------------------------------------- copies
def staged_copy(srcs, chunk_bytes: int, nslots: int):
    """P2P transfers through a staging pool: returns (dsts, events).

    events is an (n, 3) int32 array of (chunk, slot, new_state) with states
    0 idle, 1 filling, 2 draining."""
    srcs = [np.ascontiguousarray(s).view(np.uint8).ravel() for s in srcs]
    nbytes = srcs[0].size if srcs else 0
    dsts = [np.zeros_like(s) for s in srcs]
    slot_mem = np.zeros(max(1, chunk_bytes * nslots), np.uint8)
    nchunks = len(srcs) * (-(-nbytes // chunk_bytes))
    ev = np.zeros((3 * nchunks + 1, 3), np.int32)
    nev = lib().orc_staged_copy(_ptrs(srcs), _ptrs(dsts), len(srcs), nbytes, chunk_bytes,
                                nslots, slot_mem.ctypes.data, ev.ctypes.data, ev.shape[0])
    if nev < 0:
        raise ValueError("illegal staging slot transition")
    return dsts, ev[:nev]


def ring_sendrecv(sends, chunk_bytes: int, nslots: int):
    """The ring shift through the staging pool: transfer r carries send[r]
    to rank (r + 1) mod R, the transfers in order r = 0..R-1 (HOCCL §3.4,
    Fig. 6: a collective described as a group of Send/Recv pairs).  Returns
    (recvs, events) with recvs[q] the bytes rank q received."""
    R = len(sends)
    dsts, ev = staged_copy(sends, chunk_bytes, nslots)
    return [dsts[(q - 1) % R] for q in range(R)], ev


def alltoall(sends, counts, row_bytes: int):
    """counts: (R, R) rows from r to d.  Returns the R receive buffers (bytes)."""
    R = len(sends)
    counts = np.ascontiguousarray(counts, dtype=np.int64).reshape(R, R)
    sends = [np.ascontiguousarray(s).view(np.uint8).ravel() for s in sends]
    recvs = [np.zeros(int(counts[:, d].sum()) * row_bytes, np.uint8) for d in range(R)]
    _check(lib().orc_alltoall(_ptrs(sends), _ptrs(recvs), R, counts.ctypes.data, row_bytes))
    return recvs


def permute_rows(src: np.ndarray, idx: np.ndarray) -> np.ndarray:
    """dst[i, :] = src[idx[i], :] for a 2-D row-major array."""
    src = np.ascontiguousarray(src)
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    dst = np.empty((idx.size,) + src.shape[1:], src.dtype)
    row_bytes = src.itemsize * int(np.prod(src.shape[1:], dtype=np.int64))
    _check(lib().orc_permute_rows(dst.ctypes.data, src.ctypes.data, idx.ctypes.data,
                                  idx.size, src.shape[0], row_bytes))
    return dst


# ---------------------------------------------------------------------- MoE
def moe_topk(logits: np.ndarray, K: int) -> np.ndarray:
    logits = np.ascontiguousarray(logits, dtype=np.float32)
    T, E = logits.shape
    out = np.empty((T, K), np.int32)
    _check(lib().orc_moe_topk(logits.ctypes.data, T, E, K, out.ctypes.data))
    return out


def moe_plan(topk: np.ndarray, E: int, R: int):
    """Returns (src_tok, slot, cnt, ecnt) for one source rank."""
    topk = np.ascontiguousarray(topk, dtype=np.int32)
    T, K = topk.shape
    src_tok = np.empty(T * K, np.int32)
    slot = np.empty((T, K), np.int32)
    cnt = np.empty(R, np.int64)
    ecnt = np.empty(E, np.int64)
    _check(lib().orc_moe_plan(topk.ctypes.data, T, E, K, R, src_tok.ctypes.data,
                              slot.ctypes.data, cnt.ctypes.data, ecnt.ctypes.data))
    return src_tok, slot, cnt, ecnt


def moe_unpack_index(ecnt_all: np.ndarray, d: int) -> np.ndarray:
    ecnt_all = np.ascontiguousarray(ecnt_all, dtype=np.int64)
    R, E = ecnt_all.shape
    n = int(ecnt_all[:, (E // R) * d:(E // R) * (d + 1)].sum())
    out = np.empty(n, np.int32)
    _check(lib().orc_moe_unpack_index(ecnt_all.ctypes.data, R, E, d, out.ctypes.data))
    return out


def moe_dispatch(xs, topks, E: int):
    """Expert-parallel dispatch over R ranks: pack by destination, all-to-all,
    unpack to (local expert, source rank, token) order.

    xs: R arrays (T, H) of any dtype; topks: R int32 arrays (T, K).
    Returns a dict with every intermediate buffer and index."""
    R = len(xs)
    plans = [moe_plan(tk, E, R) for tk in topks]
    row_bytes = xs[0].itemsize * xs[0].shape[1]
    send = [permute_rows(x, p[0]) for x, p in zip(xs, plans)]
    counts = np.stack([p[2] for p in plans])
    ecnt = np.stack([p[3] for p in plans])
    recv_b = alltoall(send, counts, row_bytes)
    recv = [r.view(xs[0].dtype).reshape(-1, xs[0].shape[1]) for r in recv_b]
    unpack = [moe_unpack_index(ecnt, d) for d in range(R)]
    exp = [permute_rows(recv[d], unpack[d]) for d in range(R)]
    return dict(send=send, counts=counts, ecnt=ecnt, recv=recv, unpack=unpack, exp=exp,
                src_tok=[p[0] for p in plans], slot=[p[1] for p in plans])


def moe_combine(exp, plan):
    """Exact inverse of moe_dispatch: returns out[r] of shape (T, K, H) with
    out[r][t, k] = the expert row that carried token t's k-th choice."""
    R = len(exp)
    H = exp[0].shape[1]
    row_bytes = exp[0].itemsize * H
    recv = []
    for d in range(R):
        inv = np.empty_like(plan["unpack"][d])
        inv[plan["unpack"][d]] = np.arange(inv.size, dtype=np.int32)
        recv.append(permute_rows(exp[d], inv))
    back_counts = plan["counts"].T.copy()
    send_b = alltoall(recv, back_counts, row_bytes)
    send = [s.view(exp[0].dtype).reshape(-1, H) for s in send_b]
    outs = []
    for r in range(R):
        slot = plan["slot"][r]
        T, K = slot.shape
        outs.append(permute_rows(send[r], slot.reshape(-1)).reshape(T, K, H))
    return outs
