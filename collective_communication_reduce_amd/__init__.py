"""Python binding of libccr, the MI355X ring all-reduce hot path.

A thin ctypes layer over the C ABI in ``include/ccr.h``: every function here
only marshals arguments (torch tensors -> device pointers, sizes, dtype
codes, the current HIP stream) and calls the C entry point of the same name.
All of the work runs in the library's HIP kernels and SDMA copies; there is
no Python or CPU fallback, and importing this package fails loudly if the
library has not been built (``python collective_communication_reduce_amd/build.py``).

PyTorch only provides device memory (tensors) and streams.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libccr.so")

CCR_OK, CCR_ERR_INVALID_ARG, CCR_ERR_UNSUPPORTED, CCR_ERR_HIP, CCR_ERR_OOM, CCR_ERR_TIMEOUT = range(6)
CCR_F32, CCR_BF16 = 0, 1
CCR_COPY_KERNEL, CCR_COPY_SDMA = 0, 1
CCR_BF16_ACC_PER_HOP, CCR_BF16_ACC_FP32_PARTIALS = 0, 1
_STATUS = {1: "invalid argument", 2: "unsupported", 3: "HIP error", 4: "out of memory", 5: "timeout"}


class CcrError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{_STATUS.get(status, status)}: {msg}")
        self.status = status


class ccr_config_t(ctypes.Structure):
    _fields_ = [("copy_mode", ctypes.c_int32), ("cu_budget", ctypes.c_int32),
                ("slices", ctypes.c_int32), ("overlap", ctypes.c_int32),
                ("staging_chunk_bytes", ctypes.c_int64), ("staging_slots", ctypes.c_int32),
                ("bf16_acc", ctypes.c_int32), ("dma_stripe", ctypes.c_int32),
                ("dma_chunk_bytes", ctypes.c_int64), ("dma_sync", ctypes.c_int32),
                ("dma_engines", ctypes.c_int32), ("graph_cache", ctypes.c_int32),
                ("dma_deadline_us", ctypes.c_int32)]


class ccr_ring_op_t(ctypes.Structure):
    _fields_ = [("phase", ctypes.c_int32), ("slice", ctypes.c_int32), ("step", ctypes.c_int32),
                ("dst_rank", ctypes.c_int32), ("src_rank", ctypes.c_int32),
                ("chunk", ctypes.c_int32), ("lo", ctypes.c_int64), ("hi", ctypes.c_int64)]


RING_OP_DTYPE = np.dtype([("phase", np.int32), ("slice", np.int32), ("step", np.int32),
                          ("dst_rank", np.int32), ("src_rank", np.int32), ("chunk", np.int32),
                          ("lo", np.int64), ("hi", np.int64)])
STAGE_ENTRY_DTYPE = np.dtype([("stage", np.int32), ("kind", np.int32), ("src", np.int32),
                              ("dst", np.int32), ("bytes", np.int64)])
STAGE_TIME_DTYPE = np.dtype([("load", np.int64), ("bw", np.int64)])
STAGE_KINDS = ("rdma", "forward", "native")

# Every exported entry point and its argument types.
_vp, _i32, _i64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64
_SIGNATURES = {
    "ccr_config_default": [ctypes.POINTER(ccr_config_t)],
    "ccr_ctx_create": [_i32, ctypes.POINTER(ccr_config_t), ctypes.POINTER(_vp)],
    "ccr_ctx_destroy": [_vp],
    "ccr_ctx_set_config": [_vp, ctypes.POINTER(ccr_config_t)],
    "ccr_ctx_get_config": [_vp, ctypes.POINTER(ccr_config_t)],
    "ccr_ring_schedule": [_i32, _i64, _i32, _i32, _i32, _vp, _i64, ctypes.POINTER(_i64)],
    "ccr_ring_hop_layout": [_i32, _i64, _i32, _i32, _i32, _i32, _i32, _vp, _i64, ctypes.POINTER(_i64)],
    "ccr_traffic_matrix": [_vp, _i32, _vp, _vp, _vp],
    "ccr_schedule_stages": [_vp, _i32, _vp, _vp, _i64, _i64, _vp, _i64, ctypes.POINTER(_i64), _vp,
                            _i64, ctypes.POINTER(_i64)],
    "ccr_allreduce": [_vp, _vp, _i32, _i64, _i32, _vp],
    "ccr_reduce_scatter": [_vp, _vp, _i32, _i64, _i32, _vp],
    "ccr_all_gather": [_vp, _vp, _i32, _i64, _i32, _vp],
    "ccr_sendrecv": [_vp, _vp, _vp, _i32, _i64, _i32, _vp],
    "ccr_sendrecv_batch": [_vp, _vp, _vp, _i32, _i64, _vp],
    "ccr_sendrecv_batch_noalloc": [_vp, _vp, _vp, _i32, _i64, _vp],
    "ccr_alltoall": [_vp, _vp, _vp, _i32, _i64, _vp, _i32, _vp],
    "ccr_alltoall_rows": [_vp, _vp, _vp, _i32, _vp, _i64, _vp],
    "ccr_permute_rows": [_vp, _vp, _vp, _vp, _i64, _i64, _i64, _vp],
    "ccr_moe_topk": [_vp, _vp, _vp, _i64, _i32, _i32, _vp],
    "ccr_moe_plan": [_vp, _vp, _i64, _i32, _i32, _i32, _vp, _vp, _vp, _vp],
    "ccr_moe_dispatch": [_vp, _vp, _vp, _vp, _i32, _i64, _i32, _i32, _i64, _vp, _vp, _vp, _vp],
    "ccr_moe_combine": [_vp, _vp, _vp, _vp, _i32, _i64, _i32, _i32, _i64, _vp, _vp, _vp, _vp],
    "ccr_moe_dispatch_fused": [_vp, _vp, _vp, _vp, _i32, _i64, _i32, _i32, _i64, _vp, _vp],
    "ccr_moe_combine_fused": [_vp, _vp, _vp, _vp, _i32, _i64, _i32, _i32, _i64, _vp, _vp],
    "ccr_last_error": [],
    "ccr_version": [],
    "ccr_probe_cu_ids": [_vp, _vp, _i32, _vp],
    "ccr_profile_enable": [_vp, _i32],
    "ccr_profile_read": [_vp, _i32, _vp],
    "ccr_profile_intervals": [_vp, _i32, _vp, _vp, _vp, _vp, _i64, ctypes.POINTER(_i64)],
    "ccr_dma_info": [_vp, _vp, _vp],
    "ccr_dma_pace": [_i64, _i64, ctypes.c_double, _i32],
    "ccr_dma_rate": [_vp, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(_i32)],
    "ccr_sendrecv_slot_log": [_vp, _vp, _i64, ctypes.POINTER(_i64)],
    "ccr_stream_wait": [_vp, _vp, _i32],
    "ccr_dma_hold_finish": [_vp, _i32],
    "ccr_graph_cache_stats": [_vp, ctypes.POINTER(_i64), ctypes.POINTER(_i64)],
    "ccr_ctx_streams": [_vp, ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int32)],
}


def _hip_runtimes():
    """Paths of every HIP runtime library mapped into this process."""
    try:
        maps = open("/proc/self/maps").read().splitlines()
    except OSError:
        return set()
    return {l.split()[-1] for l in maps if "libamdhip64.so" in l}


def _load():
    # torch ships its own HIP runtime.  Load it first, so that libccr's
    # dependency (soname libamdhip64.so.7) resolves to that same runtime:
    # tensors, streams and libccr's kernels must share one HIP runtime.
    import torch  # noqa: F401
    import torch.cuda  # noqa: F401
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with "
            "`python collective_communication_reduce_amd/build.py` (hipcc, gfx950)")
    lib = ctypes.CDLL(LIB_PATH)
    if len(_hip_runtimes()) > 1:
        raise ImportError(f"two HIP runtimes are loaded ({sorted(_hip_runtimes())}); import "
                          "torch before anything that loads /opt/rocm's libamdhip64")
    for name, args in _SIGNATURES.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = ctypes.c_char_p if name in ("ccr_last_error", "ccr_version") else ctypes.c_int
    return lib


_lib = _load()


def _raw_stream_getter():
    import torch
    return getattr(torch._C, "_cuda_getCurrentRawStream", None)


_raw_stream = _raw_stream_getter()


def _check(status: int):
    if status != CCR_OK:
        raise CcrError(status, _lib.ccr_last_error().decode())


def ccr_version() -> str:
    return _lib.ccr_version().decode()


def ccr_last_error() -> str:
    return _lib.ccr_last_error().decode()


# ------------------------------------------------------------------ config
CCR_DMA_SYNC_HOST_FUNC, CCR_DMA_SYNC_STREAM_FLAGS = 0, 1  # ccr_dma_sync_t
_DMA_SYNC = {"host_func": CCR_DMA_SYNC_HOST_FUNC, "stream_flags": CCR_DMA_SYNC_STREAM_FLAGS}


@dataclass
class Config:
    copy_mode: str = "kernel"        # "kernel" | "sdma"
    cu_budget: int = 0               # 0 = all compute units
    slices: int = 1
    overlap: bool = False
    staging_chunk_bytes: int = 4 << 20
    staging_slots: int = 2
    bf16_acc: str = "per_hop"        # "per_hop" | "fp32_partials"
    dma_stripe: int = 0              # SDMA engines per staging copy; 0 = half of them
    dma_chunk_bytes: int = 0         # SDMA all-to-all chunk; 0 = automatic
    dma_sync: str = "host_func"      # "host_func" | "stream_flags"
    dma_engines: int = 0             # SDMA engines one call may use; 0 = all
    graph_cache: bool = True         # replay small kernel-only ring calls from captured graphs
    dma_deadline_us: int = 0         # SDMA: time a call's copies may take; > 0 paces the engines

    def to_c(self) -> ccr_config_t:
        if self.dma_sync not in _DMA_SYNC:
            raise ValueError(f"dma_sync {self.dma_sync!r} is not one of {sorted(_DMA_SYNC)}")
        return ccr_config_t(CCR_COPY_SDMA if self.copy_mode == "sdma" else CCR_COPY_KERNEL,
                            self.cu_budget, self.slices, int(self.overlap),
                            self.staging_chunk_bytes, self.staging_slots,
                            CCR_BF16_ACC_FP32_PARTIALS if self.bf16_acc == "fp32_partials"
                            else CCR_BF16_ACC_PER_HOP, self.dma_stripe, self.dma_chunk_bytes,
                            _DMA_SYNC[self.dma_sync], self.dma_engines,
                            int(self.graph_cache), self.dma_deadline_us)

    @staticmethod
    def from_c(c: ccr_config_t) -> "Config":
        return Config("sdma" if c.copy_mode == CCR_COPY_SDMA else "kernel", c.cu_budget,
                      c.slices, bool(c.overlap), c.staging_chunk_bytes, c.staging_slots,
                      "fp32_partials" if c.bf16_acc == CCR_BF16_ACC_FP32_PARTIALS else "per_hop",
                      c.dma_stripe, c.dma_chunk_bytes,
                      {v: k for k, v in _DMA_SYNC.items()}.get(c.dma_sync, "host_func"), c.dma_engines,
                      bool(c.graph_cache), c.dma_deadline_us)


def ccr_config_default() -> Config:
    c = ccr_config_t()
    _check(_lib.ccr_config_default(ctypes.byref(c)))
    return Config.from_c(c)


class Context:
    """Owns a ccr_ctx_t (side streams, events, staging slots)."""

    def __init__(self, device: int = 0, config: Optional[Config] = None):
        self.handle = ctypes.c_void_p()
        c = config.to_c() if config is not None else None
        _check(_lib.ccr_ctx_create(device, ctypes.byref(c) if c is not None else None,
                                   ctypes.byref(self.handle)))
        self.device = device

    def set_config(self, config: Config):
        c = config.to_c()
        _check(_lib.ccr_ctx_set_config(self.handle, ctypes.byref(c)))

    def config(self) -> Config:
        c = ccr_config_t()
        _check(_lib.ccr_ctx_get_config(self.handle, ctypes.byref(c)))
        return Config.from_c(c)

    def close(self):
        if self.handle:
            _check(_lib.ccr_ctx_destroy(self.handle))
            self.handle = ctypes.c_void_p()

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    def __del__(self):
        try:
            if self.handle:
                _lib.ccr_ctx_destroy(self.handle)
        except Exception:
            pass


# ------------------------------------------------------------- marshalling
def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.float32:
        return CCR_F32
    if t.dtype == torch.bfloat16:
        return CCR_BF16
    raise TypeError(f"unsupported dtype {t.dtype}; use float32 or bfloat16")


def _stream(stream) -> Optional[int]:
    import torch
    if stream is None:
        # the raw handle of the current stream, without building a Stream object
        if _raw_stream is not None:
            return _raw_stream(torch.cuda.current_device())
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else stream


def _ptrs(tensors) -> ctypes.Array:
    for t in tensors:
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError("tensors must be contiguous device tensors")
    return (ctypes.c_void_p * len(tensors))(*[t.data_ptr() for t in tensors])


def _same(tensors):
    n, dt = tensors[0].numel(), tensors[0].dtype
    if any(t.numel() != n or t.dtype != dt for t in tensors):
        raise ValueError("all ranks need the same element count and dtype")
    return n


def _ring_args(bufs):
    """(pointer array, count, dtype code) of R same-shaped contiguous device
    tensors, in one pass."""
    t0 = bufs[0]
    n, dt = t0.numel(), t0.dtype
    ptrs = (ctypes.c_void_p * len(bufs))()
    for i, t in enumerate(bufs):
        if t.numel() != n or t.dtype != dt:
            raise ValueError("all ranks need the same element count and dtype")
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError("tensors must be contiguous device tensors")
        ptrs[i] = t.data_ptr()
    return ptrs, n, _dtype_code(t0)


# --------------------------------------------------------------- C entries
def ccr_ring_schedule(R: int, count: int, slices: int, dtype: int, which: int = 0) -> np.ndarray:
    n = ctypes.c_int64()
    _check(_lib.ccr_ring_schedule(R, count, slices, dtype, which, None, 0, ctypes.byref(n)))
    out = np.zeros(n.value, RING_OP_DTYPE)
    _check(_lib.ccr_ring_schedule(R, count, slices, dtype, which,
                                  out.ctypes.data if n.value else None, n.value, ctypes.byref(n)))
    return out


def ccr_ring_hop_layout(R: int, count: int, slices: int, dtype: int, phase: int, step: int,
                        slice: int = 0) -> np.ndarray:
    """[workgroups x 5] int64: source rank, destination rank, byte offset and
    byte length of the piece, tile index -- per workgroup of one ring-hop
    launch, as the kernel maps them."""
    n = ctypes.c_int64()
    _check(_lib.ccr_ring_hop_layout(R, count, slices, dtype, phase, step, slice, None, 0,
                                    ctypes.byref(n)))
    out = np.zeros((n.value, 5), np.int64)
    _check(_lib.ccr_ring_hop_layout(R, count, slices, dtype, phase, step, slice,
                                    out.ctypes.data if n.value else None, n.value, ctypes.byref(n)))
    return out


def _schedule_args(C, node, peer):
    C = np.ascontiguousarray(C, dtype=np.int64)
    G = C.shape[0]
    if C.ndim != 2 or C.shape[1] != G:
        raise ValueError("C must be a square G x G matrix")
    node = np.ascontiguousarray(node, dtype=np.int32)
    peer = np.ascontiguousarray(peer, dtype=np.int32)
    if node.shape != (G,) or peer.shape != (G,):
        raise ValueError("node and peer need one entry per GPU")
    return C, G, node, peer


def ccr_traffic_matrix(C, node, peer) -> np.ndarray:
    """T (G x G int64) from the origin traffic matrix C."""
    C, G, node, peer = _schedule_args(C, node, peer)
    T = np.zeros((G, G), np.int64)
    _check(_lib.ccr_traffic_matrix(C.ctypes.data, G, node.ctypes.data, peer.ctypes.data,
                                   T.ctypes.data))
    return T


def ccr_schedule_stages(C, node, peer, bw_scaleup: int, bw_rdma: int):
    """(entries, times): the stage records (STAGE_ENTRY_DTYPE) and each
    stage's time as load / bw (STAGE_TIME_DTYPE)."""
    C, G, node, peer = _schedule_args(C, node, peer)
    ne, ns = ctypes.c_int64(), ctypes.c_int64()
    args = (C.ctypes.data, G, node.ctypes.data, peer.ctypes.data, bw_scaleup, bw_rdma)
    # Room for a typical schedule, so that one call usually suffices; call
    # again with the exact sizes when it does not.
    cap_s = G * G + 16
    cap_e = min(cap_s * (3 * G + 8), 1 << 20)
    while True:
        entries = np.empty(cap_e, STAGE_ENTRY_DTYPE)
        times = np.empty(cap_s, STAGE_TIME_DTYPE)
        _check(_lib.ccr_schedule_stages(*args, entries.ctypes.data, cap_e, ctypes.byref(ne),
                                        times.ctypes.data, cap_s, ctypes.byref(ns)))
        if ne.value <= cap_e and ns.value <= cap_s:
            return entries[:ne.value].copy(), times[:ns.value].copy()
        cap_e, cap_s = ne.value, ns.value


def ccr_allreduce(ctx: Context, bufs: Sequence, stream=None):
    ptrs, n, dt = _ring_args(bufs)
    _check(_lib.ccr_allreduce(ctx.handle, ptrs, len(bufs), n, dt, _stream(stream)))


def ccr_reduce_scatter(ctx: Context, bufs: Sequence, stream=None):
    ptrs, n, dt = _ring_args(bufs)
    _check(_lib.ccr_reduce_scatter(ctx.handle, ptrs, len(bufs), n, dt, _stream(stream)))


def ccr_all_gather(ctx: Context, bufs: Sequence, stream=None):
    ptrs, n, dt = _ring_args(bufs)
    _check(_lib.ccr_all_gather(ctx.handle, ptrs, len(bufs), n, dt, _stream(stream)))


def ccr_sendrecv(ctx: Context, send: Sequence, recv: Sequence, stream=None):
    """Ring shift: recv[(r + 1) % R] <- send[r] for the R = len(send) ranks."""
    if len(send) != len(recv) or not send:
        raise ValueError("send and recv need one buffer per rank")
    ptrs, n, dt = _ring_args(list(send))
    rp, rn, rdt = _ring_args(list(recv))
    if rn != n or rdt != dt:
        raise ValueError("send and recv buffers need the same element count and dtype")
    _check(_lib.ccr_sendrecv(ctx.handle, ptrs, rp, len(send), n, dt, _stream(stream)))


def ccr_sendrecv_batch(ctx: Context, send: Sequence, recv: Sequence, stream=None):
    """recv[m] <- send[m] for every transfer m, in order."""
    if len(send) != len(recv):
        raise ValueError("send and recv need the same number of transfers")
    nbytes = send[0].numel() * send[0].element_size() if send else 0
    if any(t.numel() * t.element_size() != nbytes for t in list(send) + list(recv)):
        raise ValueError("every transfer moves the same number of bytes")
    _check(_lib.ccr_sendrecv_batch(ctx.handle, _ptrs(send), _ptrs(recv), len(send), nbytes,
                                   _stream(stream)))


def ccr_sendrecv_batch_noalloc(ctx: Context, send: Sequence, recv: Sequence, stream=None):
    """ccr_sendrecv_batch staged through the GPU's fixed 16 MiB scratch: no
    allocation (kernel copies; slots x chunk <= 16 MiB)."""
    if len(send) != len(recv):
        raise ValueError("send and recv need the same number of transfers")
    nbytes = send[0].numel() * send[0].element_size() if send else 0
    if any(t.numel() * t.element_size() != nbytes for t in list(send) + list(recv)):
        raise ValueError("every transfer moves the same number of bytes")
    _check(_lib.ccr_sendrecv_batch_noalloc(ctx.handle, _ptrs(send), _ptrs(recv), len(send), nbytes,
                                           _stream(stream)))


def ccr_alltoall(ctx: Context, send: Sequence, recv: Sequence, counts=None, stream=None):
    """send[r] holds count elements (its segments in destination order);
    counts[r][d] elements go from r to d, or count / R each when counts is
    None; recv[d] gets its segments in source order."""
    R = len(send)
    if len(recv) != R:
        raise ValueError("send and recv need one buffer per rank")
    ptrs, n, dt = _ring_args(list(send))
    c = None
    if counts is not None:
        c = np.ascontiguousarray(counts, dtype=np.int64).reshape(R, R)
    _check(_lib.ccr_alltoall(ctx.handle, ptrs, _ptrs(recv), R, n,
                             c.ctypes.data if c is not None else None, dt, _stream(stream)))


def ccr_alltoall_rows(ctx: Context, send: Sequence, recv: Sequence, counts, row_bytes: int,
                      stream=None):
    """counts[r][d] rows of row_bytes from rank r to rank d."""
    R = len(send)
    counts = np.ascontiguousarray(counts, dtype=np.int64).reshape(R, R)
    _check(_lib.ccr_alltoall_rows(ctx.handle, _ptrs(send), _ptrs(recv), R, counts.ctypes.data,
                                  row_bytes, _stream(stream)))


def ccr_permute_rows(ctx: Context, dst, src, idx, stream=None):
    row_bytes = (src.numel() // max(1, src.shape[0])) * src.element_size()
    _check(_lib.ccr_permute_rows(ctx.handle, dst.data_ptr(), src.data_ptr(), idx.data_ptr(),
                                 idx.numel(), src.shape[0], row_bytes, _stream(stream)))


def ccr_moe_topk(ctx: Context, logits, topk, stream=None):
    T, E = logits.shape
    _check(_lib.ccr_moe_topk(ctx.handle, logits.data_ptr(), topk.data_ptr(), T, E,
                             topk.shape[1], _stream(stream)))


def ccr_moe_plan(ctx: Context, topk, E: int, R: int, src_tok, slot, stream=None) -> np.ndarray:
    """Blocking: returns the host int64 [E] row counts per expert."""
    T, K = topk.shape
    ecnt = np.zeros(E, np.int64)
    _check(_lib.ccr_moe_plan(ctx.handle, topk.data_ptr(), T, E, K, R, src_tok.data_ptr(),
                             slot.data_ptr(), ecnt.ctypes.data, _stream(stream)))
    return ecnt


def ccr_moe_dispatch(ctx: Context, x: Sequence, src_tok: Sequence, ecnt, K: int,
                     send: Sequence, recv: Sequence, exp: Sequence, stream=None):
    R = len(x)
    T = x[0].shape[0]
    row_bytes = x[0].shape[-1] * x[0].element_size()
    ecnt = np.ascontiguousarray(ecnt, dtype=np.int64)
    _check(_lib.ccr_moe_dispatch(ctx.handle, _ptrs(x), _ptrs(src_tok), ecnt.ctypes.data, R, T,
                                 ecnt.shape[1], K, row_bytes, _ptrs(send), _ptrs(recv),
                                 _ptrs(exp), _stream(stream)))


def ccr_moe_combine(ctx: Context, exp: Sequence, slot: Sequence, ecnt, T: int, K: int,
                    recv: Sequence, send: Sequence, out: Sequence, stream=None):
    R = len(exp)
    row_bytes = exp[0].shape[-1] * exp[0].element_size()
    ecnt = np.ascontiguousarray(ecnt, dtype=np.int64)
    _check(_lib.ccr_moe_combine(ctx.handle, _ptrs(exp), _ptrs(slot), ecnt.ctypes.data, R, T,
                                ecnt.shape[1], K, row_bytes, _ptrs(recv), _ptrs(send),
                                _ptrs(out), _stream(stream)))


def ccr_moe_dispatch_fused(ctx: Context, x: Sequence, src_tok: Sequence, ecnt, K: int,
                           exp: Sequence, stream=None):
    R = len(x)
    T = x[0].shape[0]
    row_bytes = x[0].shape[-1] * x[0].element_size()
    ecnt = np.ascontiguousarray(ecnt, dtype=np.int64)
    _check(_lib.ccr_moe_dispatch_fused(ctx.handle, _ptrs(x), _ptrs(src_tok), ecnt.ctypes.data, R,
                                       T, ecnt.shape[1], K, row_bytes, _ptrs(exp), _stream(stream)))


def ccr_moe_combine_fused(ctx: Context, exp: Sequence, slot: Sequence, ecnt, T: int, K: int,
                          out: Sequence, stream=None):
    R = len(exp)
    row_bytes = out[0].shape[-1] * out[0].element_size()
    ecnt = np.ascontiguousarray(ecnt, dtype=np.int64)
    _check(_lib.ccr_moe_combine_fused(ctx.handle, _ptrs(exp), _ptrs(slot), ecnt.ctypes.data, R, T,
                                      ecnt.shape[1], K, row_bytes, _ptrs(out), _stream(stream)))


def ccr_probe_cu_ids(ctx: Context, nblocks: int, stream=None):
    """(nblocks, 3) int32 tensor of (XCC id, SE id, CU id) per workgroup."""
    import torch
    out = torch.zeros(nblocks, 3, dtype=torch.int32, device=f"cuda:{ctx.device}")
    _check(_lib.ccr_probe_cu_ids(ctx.handle, out.data_ptr(), nblocks, _stream(stream)))
    return out


class ccr_kernel_stats_t(ctypes.Structure):
    _fields_ = [("launches", ctypes.c_int64), ("bytes", ctypes.c_int64), ("ms", ctypes.c_double)]


PROFILE_KINDS = {"reduce": 0, "copy_kernel": 1, "sdma": 2, "reduce_forward": 3, "moe_gather": 4}


def ccr_profile_enable(ctx: Context, on: bool = True):
    _check(_lib.ccr_profile_enable(ctx.handle, int(on)))


def ccr_profile_read(ctx: Context, kind: str) -> dict:
    st = ccr_kernel_stats_t()
    _check(_lib.ccr_profile_read(ctx.handle, PROFILE_KINDS[kind], ctypes.byref(st)))
    return {"launches": st.launches, "bytes": st.bytes, "ms": st.ms}


def ccr_profile_intervals(ctx: Context, kind: str, ref_event) -> np.ndarray:
    """(n, 3) float64 array of (start ms, end ms, compute units held) of
    every timed launch of `kind`, relative to the recorded torch.cuda.Event
    `ref_event` (created with enable_timing=True)."""
    n = ctypes.c_int64()
    ref = ctypes.c_void_p(ref_event.cuda_event)
    _check(_lib.ccr_profile_intervals(ctx.handle, PROFILE_KINDS[kind], ref, None, None, None, 0,
                                      ctypes.byref(n)))
    a = np.zeros(n.value, np.float64)
    b = np.zeros(n.value, np.float64)
    c = np.zeros(n.value, np.int32)
    if n.value:
        _check(_lib.ccr_profile_intervals(ctx.handle, PROFILE_KINDS[kind], ref, a.ctypes.data,
                                          b.ctypes.data, c.ctypes.data, n.value, ctypes.byref(n)))
    return np.stack([a, b, c.astype(np.float64)], axis=1) if n.value else np.zeros((0, 3))


def ccr_dma_info(ctx: Context) -> list:
    """HSA indices of the SDMA engines the context's DMA proxy uses."""
    n = ctypes.c_int32()
    ids = (ctypes.c_int32 * 16)()
    _check(_lib.ccr_dma_info(ctx.handle, ctypes.byref(n), ids))
    return list(ids[:n.value])


def ccr_dma_pace(nbytes: int, deadline_us: int, engine_gbs: float, max_engines: int) -> int:
    """Fewest SDMA engines that move nbytes within deadline_us at engine_gbs each (host only)."""
    return int(_lib.ccr_dma_pace(nbytes, deadline_us, engine_gbs, max_engines))


def ccr_dma_rate(ctx: Context) -> tuple:
    """(one engine's measured copy rate in GB/s, engines the last SDMA job was allowed)."""
    g, e = ctypes.c_double(), ctypes.c_int32()
    _check(_lib.ccr_dma_rate(ctx.handle, ctypes.byref(g), ctypes.byref(e)))
    return g.value, e.value


def ccr_sendrecv_slot_log(ctx: Context) -> np.ndarray:
    """(n, 3) int32 array of (chunk, slot, new state) of the last SDMA staged transfer."""
    n = ctypes.c_int64()
    _check(_lib.ccr_sendrecv_slot_log(ctx.handle, None, 0, ctypes.byref(n)))
    out = np.zeros((n.value, 3), np.int32)
    if n.value:
        _check(_lib.ccr_sendrecv_slot_log(ctx.handle, out.ctypes.data, n.value, ctypes.byref(n)))
    return out


def ccr_stream_wait(ctx: Context, timeout_ms: int, stream=None) -> int:
    """Returns CCR_OK or CCR_ERR_TIMEOUT; raises on other errors."""
    st = _lib.ccr_stream_wait(ctx.handle, _stream(stream), timeout_ms)
    if st not in (CCR_OK, CCR_ERR_TIMEOUT):
        _check(st)
    return st


def ccr_dma_hold_finish(ctx: Context, us: int):
    _check(_lib.ccr_dma_hold_finish(ctx.handle, us))


def ccr_graph_cache_stats(ctx: Context) -> tuple:
    """(graphs held, ring calls served by a replay so far)."""
    g, r = ctypes.c_int64(), ctypes.c_int64()
    _check(_lib.ccr_graph_cache_stats(ctx.handle, ctypes.byref(g), ctypes.byref(r)))
    return g.value, r.value


def ccr_ctx_streams(ctx: Context) -> tuple:
    """(CU-masked side streams, plain streams) the context holds now."""
    m, p = ctypes.c_int32(), ctypes.c_int32()
    _check(_lib.ccr_ctx_streams(ctx.handle, ctypes.byref(m), ctypes.byref(p)))
    return m.value, p.value
