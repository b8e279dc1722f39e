"""The library's stage scheduler (host code behind the C ABI) against the
oracle: integer results, compared exactly."""
import ctypes

import numpy as np
import pytest

import collective_communication_reduce_amd as ccr
from oracle import collective_schedule as cs
import workloads as W


def _oracle(C, node, peer, bnv, brd):
    st = cs.decompose(C, node, peer, bnv, brd)
    entries = [(s, k, u, v, b) for s, x in enumerate(st) for k, u, v, b in x["entries"]]
    return entries, [x["tau"] for x in st]


def _lib(C, node, peer, bnv, brd):
    e, t = ccr.ccr_schedule_stages(C, node, peer, bnv, brd)
    return [tuple(int(x) for x in r) for r in e.tolist()], [tuple(int(x) for x in r) for r in t.tolist()]


def _cases():
    topos = [
        W.FIG6_TOPOLOGY,
        W.Topology("2x4", 2, 4, 5, 2),
        W.Topology("2x8", 2, 8, 153, 50),
        W.Topology("4x4", 4, 4, 7, 3),
        W.Topology("4x8", 4, 8, 153, 50),
        W.Topology("3x2_unpaired", 3, 2, 4, 1, paired=False),
        W.Topology("1x8", 1, 8, 153, 50),
        W.Topology("8x1", 8, 1, 1, 1, paired=False),
        W.Topology("2x8_equal_bw", 2, 8, 1, 1),
    ]
    for t in topos:
        for seed, (dens, top) in enumerate([(0.3, 1000), (0.7, 10), (1.0, 1 << 30), (0.5, 3)]):
            yield f"{t.name}-{seed}", t.G, t.node(), t.peer(), t.bw_scaleup, t.bw_rdma, \
                W.random_traffic(t.G, [21, t.G, seed], top, density=dens)


CASES = list(_cases())


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_schedule_matches_oracle(case):
    _, G, node, peer, bnv, brd, C = case
    assert _lib(C, node, peer, bnv, brd) == _oracle(C, node, peer, bnv, brd)
    assert ccr.ccr_traffic_matrix(C, node, peer).tolist() == cs.traffic_matrix(C, node, peer)


def test_moe_dispatch_traffic_matches_oracle():
    w = W.SCHED_MOE_2X8
    t = w.topology
    C = W.moe_traffic(w)
    assert _lib(C, t.node(), t.peer(), t.bw_scaleup, t.bw_rdma) == \
        _oracle(C, t.node(), t.peer(), t.bw_scaleup, t.bw_rdma)


def test_unsorted_node_ids_and_uneven_nodes():
    # nodes named 7, 3, 0 in no order, of sizes 3, 2, 3; peers only in some
    node = [7, 3, 7, 0, 3, 0, 7, 0]
    peer = [2, 4, 0, -1, 1, 7, -1, 5]
    for seed in range(6):
        C = W.random_traffic(8, [31, seed], 97, density=0.8)
        assert _lib(C, node, peer, 11, 4) == _oracle(C, node, peer, 11, 4)
        assert ccr.ccr_traffic_matrix(C, node, peer).tolist() == cs.traffic_matrix(C, node, peer)


def test_golden_figure6_example():
    C = [[0] * 4 for _ in range(4)]
    C[0][2], C[1][3], C[0][3], C[0][1], C[2][3] = 4, 2, 1, 6, 3
    e, t = _lib(C, [0, 0, 1, 1], [1, 0, 3, 2], 3, 1)
    assert t == [(2, 1), (2, 1), (1, 1)]
    assert e[:8] == [(0, 0, 0, 2, 2), (0, 0, 1, 3, 2), (0, 1, 0, 1, 2), (0, 1, 1, 0, 2),
                     (0, 1, 2, 3, 2), (0, 1, 3, 2, 2), (0, 2, 0, 1, 4), (0, 2, 2, 3, 3)]


def test_empty_single_gpu_and_diagonal():
    assert _lib([[0]], [0], [-1], 1, 1) == ([], [])
    assert _lib([[5]], [0], [-1], 1, 1) == ([], [])  # the diagonal is not traffic
    Z = np.zeros((4, 4), np.int64)
    assert _lib(Z, [0, 0, 1, 1], [1, 0, 3, 2], 3, 1) == ([], [])
    assert ccr.ccr_traffic_matrix(np.full((3, 3), 9), [0, 0, 0], [-1, -1, -1]).tolist() == \
        [[0, 9, 9], [9, 0, 9], [9, 9, 0]]


def test_largest_values_stay_exact():
    """Flows at the 2^40-byte limit and bandwidths at 2^20: products need
    more than 64 bits in the stage-time comparison."""
    big = 1 << 40
    C = [[0, big, big, big - 1], [big, 0, 1, big], [big, 3, 0, big], [big - 7, big, big, 0]]
    for bnv, brd in [(1 << 20, 1), (1, 1 << 20), (1 << 20, (1 << 20) - 1)]:
        assert _lib(C, [0, 0, 1, 1], [1, 0, 3, 2], bnv, brd) == \
            _oracle(C, [0, 0, 1, 1], [1, 0, 3, 2], bnv, brd)


def test_truncated_output_reports_full_counts():
    w = W.SCHED_MOE_2X8
    t = w.topology
    C = np.ascontiguousarray(W.moe_traffic(w), np.int64)
    node = np.array(t.node(), np.int32)
    peer = np.array(t.peer(), np.int32)
    full_e, full_t = ccr.ccr_schedule_stages(C, node, peer, t.bw_scaleup, t.bw_rdma)
    part_e = np.zeros(5, ccr.STAGE_ENTRY_DTYPE)
    part_t = np.zeros(2, ccr.STAGE_TIME_DTYPE)
    ne, ns = ctypes.c_int64(), ctypes.c_int64()
    st = ccr._lib.ccr_schedule_stages(C.ctypes.data, t.G, node.ctypes.data, peer.ctypes.data,
                                      t.bw_scaleup, t.bw_rdma, part_e.ctypes.data, 5,
                                      ctypes.byref(ne), part_t.ctypes.data, 2, ctypes.byref(ns))
    assert st == ccr.CCR_OK
    assert (ne.value, ns.value) == (len(full_e), len(full_t))
    assert part_e.tolist() == full_e[:5].tolist() and part_t.tolist() == full_t[:2].tolist()


@pytest.mark.parametrize("bad", [
    dict(node=[0, 0, 1, -1]),                 # negative node id
    dict(peer=[1, 0, 3, 3]),                  # own peer
    dict(peer=[2, 0, 3, 2]),                  # peer in another node
    dict(peer=[1, 0, 3, 9]),                  # out of range
    dict(peer=[1, -1, 3, 2]),                 # not mutual (0 names 1, 1 names nobody)
    dict(node=[0, 0, 0, 1], peer=[1, 2, 0, -1]),  # not mutual (a cycle)
    dict(C_fix=(0, 1, -5)),                   # negative bytes
    dict(C_fix=(0, 1, (1 << 40) + 1)),        # above the limit
    dict(bw=(0, 1)),
    dict(bw=(1, (1 << 20) + 1)),
])
def test_invalid_arguments(bad):
    C = [[0, 1, 2, 3], [1, 0, 2, 3], [1, 2, 0, 3], [1, 2, 3, 0]]
    if "C_fix" in bad:
        u, v, b = bad["C_fix"]
        C[u][v] = b
    node = bad.get("node", [0, 0, 1, 1])
    peer = bad.get("peer", [1, 0, 3, 2])
    bnv, brd = bad.get("bw", (3, 1))
    with pytest.raises(ccr.CcrError) as ei:
        ccr.ccr_schedule_stages(C, node, peer, bnv, brd)
    assert ei.value.status == ccr.CCR_ERR_INVALID_ARG
    if "bw" not in bad:
        with pytest.raises(ccr.CcrError):
            ccr.ccr_traffic_matrix(C, node, peer)


def test_null_and_size_arguments():
    one = (ctypes.c_int64 * 1)(0)
    i32 = (ctypes.c_int32 * 1)(0)
    m1 = (ctypes.c_int32 * 1)(-1)
    n = ctypes.c_int64()
    lib = ccr._lib
    assert lib.ccr_traffic_matrix(None, 1, i32, m1, one) == ccr.CCR_ERR_INVALID_ARG
    assert lib.ccr_traffic_matrix(one, 1, i32, m1, None) == ccr.CCR_ERR_INVALID_ARG
    assert lib.ccr_traffic_matrix(one, 0, i32, m1, one) == ccr.CCR_ERR_INVALID_ARG
    assert lib.ccr_traffic_matrix(one, 257, i32, m1, one) == ccr.CCR_ERR_INVALID_ARG
    assert lib.ccr_schedule_stages(one, 1, i32, m1, 1, 1, None, 0, None, None, 0,
                                   ctypes.byref(n)) == ccr.CCR_ERR_INVALID_ARG
    assert lib.ccr_schedule_stages(one, 1, i32, m1, 1, 1, None, -1, ctypes.byref(n), None, 0,
                                   ctypes.byref(n)) == ccr.CCR_ERR_INVALID_ARG
    assert "NULL" in ccr.ccr_last_error() or "negative" in ccr.ccr_last_error()
