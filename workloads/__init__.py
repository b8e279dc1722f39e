"""Seeded synthetic inputs shared by the GPU tests, the oracle tests and the
benchmark.

This module only draws random numbers and shapes them; it holds none of the
collective's arithmetic.  Values are drawn with numpy's PCG64
(``default_rng([seed, index])``) in float64, rounded to float32, and -- for
bfloat16 buffers -- converted to bf16 by torch's own float32->bfloat16 cast
(round to nearest even).  bf16 buffers are carried as uint16 arrays of the
raw bits.

The workloads stand in for the traffic the HOCCL paper measures ("HOCCL:
Offloading Collective Communication from GPU Cores to Accelerate Distributed
Training", §2.1 Distributed Training Workloads; §6.1 Experiment Setup, Table 2;
§6.2 Communication Benchmark): data-parallel gradient buckets, pipeline-
parallel activations of the 6.7B model (sequence 2048 x hidden 4096) and
expert-parallel token dispatch.  No dataset, model weight or benchmark suite
is used.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

MiB = 1 << 20


@dataclass(frozen=True)
class RingWorkload:
    name: str
    R: int           # virtual ranks
    count: int       # elements per rank
    dtype: str       # "f32" or "bf16"
    dist: str        # "uniform" (on [-1, 1]) or "normal"
    scale: float     # std of the normal draw
    seed: int
    slices: int      # pipeline slices per chunk


# Ring all-reduce, 4 ranks x 1,048,576 fp32, uniform[-1, 1], 2 slices per chunk.
RING_SMALL_F32 = RingWorkload("ring_allreduce_r4_1m_f32", 4, 1 << 20, "f32", "uniform", 1.0, 1, 2)
# Data-parallel gradient bucket: 8 ranks x 25 Mi bf16 (50 MiB), normal(0, 1e-3).
DP_BUCKET_BF16 = RingWorkload("dp_bucket_allreduce_r8_25m_bf16", 8, 25 * MiB, "bf16", "normal", 1e-3, 2, 1)
# Reduce-scatter then all-gather, 32 ranks x 8 Mi fp32 (1 GiB in total).
RS_AG_R32_F32 = RingWorkload("rs_ag_r32_8m_f32", 32, 8 * MiB, "f32", "uniform", 1.0, 4, 4)

RING_WORKLOADS = (RING_SMALL_F32, DP_BUCKET_BF16, RS_AG_R32_F32)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bits via torch's cast (round to nearest even)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def draw(seed, n: int, dist: str, scale: float = 1.0) -> np.ndarray:
    """n float32 values from default_rng(seed)."""
    rng = np.random.default_rng(seed)
    if dist == "uniform":
        v = rng.uniform(-1.0, 1.0, n)
    elif dist == "normal":
        v = rng.normal(0.0, scale, n)
    else:
        raise ValueError(dist)
    return v.astype(np.float32)


def ring_inputs(w: RingWorkload, count: int | None = None, R: int | None = None):
    """Per-rank input buffers of a ring workload (optionally resized)."""
    n = w.count if count is None else count
    R = w.R if R is None else R
    out = []
    for r in range(R):
        v = draw([w.seed, r], n, w.dist, w.scale)
        out.append(f32_to_bf16_bits(v) if w.dtype == "bf16" else v)
    return out


def random_buffers(R: int, n: int, dtype: str, seed: int, dist: str = "uniform",
                   scale: float = 1.0):
    """Small ad-hoc per-rank buffers for tests."""
    out = []
    for r in range(R):
        v = draw([seed, r], n, dist, scale)
        out.append(f32_to_bf16_bits(v) if dtype == "bf16" else v)
    return out


def integer_buffers(R: int, n: int, dtype: str, seed: int, bound: int):
    """Per-rank buffers of integers in [-bound, bound] (exact in fp32/bf16 for
    small bounds), so that any summation order gives the same exact sum."""
    rng = np.random.default_rng([seed, 77])
    out = []
    for _ in range(R):
        v = rng.integers(-bound, bound + 1, n).astype(np.float32)
        out.append(f32_to_bf16_bits(v) if dtype == "bf16" else v)
    return out


# ------------------------------------------------------------- PP staging
@dataclass(frozen=True)
class StagingWorkload:
    name: str
    microbatches: int
    rows: int          # sequence length
    cols: int          # hidden size
    chunk_bytes: int
    slots: int
    seed: int


# Pipeline activations of the 6.7B model (seq 2048 x hidden 4096, bf16),
# 4 micro-batches, moved in 4 MiB chunks through 2 staging slots.
PP_STAGING_BF16 = StagingWorkload("pp_sendrecv_4x2048x4096_bf16", 4, 2048, 4096, 4 * MiB, 2, 3)


def staging_inputs(w: StagingWorkload, rows: int | None = None):
    rows = w.rows if rows is None else rows
    return [f32_to_bf16_bits(draw([w.seed, m], rows * w.cols, "normal", 1.0)).reshape(rows, w.cols)
            for m in range(w.microbatches)]


# ------------------------------------------------------------- MoE dispatch
@dataclass(frozen=True)
class MoeWorkload:
    name: str
    R: int
    tokens: int
    hidden: int
    experts: int
    topk: int
    seed: int


# Expert-parallel dispatch: 8 ranks x 4096 tokens x 2048 hidden bf16,
# 64 experts (8 per rank), top-6 routing over normal(0, 1) logits.
MOE_DISPATCH_BF16 = MoeWorkload("moe_dispatch_r8_4096x2048_bf16_e64_top6", 8, 4096, 2048, 64, 6, 5)


def moe_inputs(w: MoeWorkload, tokens: int | None = None, R: int | None = None):
    """(xs, logits): per-rank activations (bf16 bits, T x H) and router
    logits (float32, T x E)."""
    T = w.tokens if tokens is None else tokens
    R = w.R if R is None else R
    xs = [f32_to_bf16_bits(draw([w.seed, r], T * w.hidden, "normal", 1.0)).reshape(T, w.hidden)
          for r in range(R)]
    logits = [draw([w.seed, 1000 + r], T * w.experts, "normal", 1.0).reshape(T, w.experts)
              for r in range(R)]
    return xs, logits


# ------------------------------------------------------------- stage schedule
@dataclass(frozen=True)
class Topology:
    """A modelled cluster: `nodes` scale-up domains of `gpus_per_node` GPUs.
    Bandwidths are integers in bytes per nanosecond (GB/s): one scale-up
    link, one NIC.  With `paired`, GPUs 2i and 2i+1 of a node are symmetric
    peers that stage each other's inter-node traffic; otherwise no GPU
    forwards."""
    name: str
    nodes: int
    gpus_per_node: int
    bw_scaleup: int
    bw_rdma: int
    paired: bool = True

    @property
    def G(self) -> int:
        return self.nodes * self.gpus_per_node

    def node(self) -> list[int]:
        return [u // self.gpus_per_node for u in range(self.G)]

    def peer(self) -> list[int]:
        return [u ^ 1 for u in range(self.G)] if self.paired else [-1] * self.G


# Figure 6 of the HOCCL paper: two nodes of two GPUs, peers 0<->1, 2<->3.
FIG6_TOPOLOGY = Topology("fig6_2x2", 2, 2, 3, 1)
# Two nodes of eight MI355X: one xGMI link carries about 153 GB/s per
# direction, one 400 Gb/s NIC about 50 GB/s.
MI355X_2X8 = Topology("mi355x_2x8_xgmi153_nic50", 2, 8, 153, 50)


@dataclass(frozen=True)
class ScheduleWorkload:
    name: str
    topology: Topology
    tokens: int
    hidden: int
    topk: int
    skew: float        # Zipf exponent of destination popularity
    seed: int


# Expert-parallel dispatch traffic across 16 GPUs: each GPU sends
# tokens x topk rows of `hidden` bf16 values, spread over destinations with
# Zipf-skewed popularity (the long-tail flows of an MoE all-to-all).
SCHED_MOE_2X8 = ScheduleWorkload("stage_schedule_moe_dispatch_2x8_4096x2048_bf16_top6",
                                 MI355X_2X8, 4096, 2048, 6, 1.2, 7)


def random_traffic(G: int, seed, max_bytes: int, density: float = 0.7) -> list[list[int]]:
    """A G x G origin traffic matrix of integers in [1, max_bytes] on about
    `density` of the off-diagonal pairs, zero elsewhere."""
    rng = np.random.default_rng(seed)
    vals = rng.integers(1, max_bytes + 1, size=(G, G))
    keep = rng.random((G, G)) < density
    return [[int(vals[u, v]) if (keep[u, v] and u != v) else 0 for v in range(G)] for u in range(G)]


def moe_traffic(w: ScheduleWorkload) -> list[list[int]]:
    """Origin traffic matrix (bytes) of one skewed dispatch: source u sends
    counts[u][v] rows of hidden bf16 values to v, counts multinomial over a
    Zipf popularity that each source permutes with its own draw."""
    G = w.topology.G
    rng = np.random.default_rng([w.seed, 0])
    base = 1.0 / np.arange(1, G + 1) ** w.skew
    C = []
    for u in range(G):
        p = rng.permutation(base)
        p = p / p.sum()
        counts = rng.multinomial(w.tokens * w.topk, p)
        C.append([int(counts[v]) * w.hidden * 2 if v != u else 0 for v in range(G)])
    return C
