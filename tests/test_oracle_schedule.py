"""Pins of the stage-decomposition oracle against what the HOCCL paper's
§3.4 (Figure 6, Eq. 2-11, Algorithm 1) and the mathematics fix."""
import itertools
import os

import pytest

from oracle import collective_schedule as cs
import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")

TOPOLOGIES = [
    W.FIG6_TOPOLOGY,
    W.Topology("2x4", 2, 4, 5, 2),
    W.Topology("2x8", 2, 8, 153, 50),
    W.Topology("4x4", 4, 4, 7, 3),
    W.Topology("3x2_unpaired", 3, 2, 4, 1, paired=False),
    W.Topology("1x8", 1, 8, 153, 50),
]


def _check_cases():
    for t in TOPOLOGIES:
        for seed in range(4):
            yield t, W.random_traffic(t.G, [11, t.G, seed], 1000, density=(0.3, 0.7, 1.0, 0.5)[seed])


CASES = list(_check_cases())


def _rdma(t, u, v):
    return t.node()[u] != t.node()[v]


def test_figure6_cell_f1():
    """Eq. 5's worked cell: on Figure 6's topology T[0,1] carries the native
    flow f1, g0's sender-side copies of f2 and f3, and the receiver-side
    copies of f8 and f11 (the flows that end at g1).  Flows f1..f12 fill C
    row by row, skipping the diagonal; each is a distinct power of two, so
    the sum names exactly which flows a cell holds."""
    G = 4
    C = [[0] * G for _ in range(G)]
    f = {}
    i = 1
    for u in range(G):
        for v in range(G):
            if u != v:
                C[u][v] = f[i] = 1 << i
                i += 1
    assert C[0][1] == f[1] and C[0][2] == f[2] and C[3][2] == f[12]  # as printed
    t = W.FIG6_TOPOLOGY
    T = cs.traffic_matrix(C, t.node(), t.peer())
    assert T[0][1] == f[1] + f[2] + f[3] + f[8] + f[11]
    # the other three scale-up cells, by the same rule
    assert T[1][0] == f[4] + f[5] + f[6] + f[7] + f[10]
    assert T[2][3] == f[9] + f[7] + f[8] + f[3] + f[6]
    assert T[3][2] == f[12] + f[10] + f[11] + f[2] + f[5]
    for u, v in itertools.product(range(G), range(G)):
        if _rdma(t, u, v):
            assert T[u][v] == C[u][v]  # RDMA entries are the logical flows
    assert all(T[u][u] == 0 for u in range(G))


def _read_golden(name):
    C, stages, taus, topo = None, {}, {}, None
    with open(os.path.join(GOLDEN, name)) as fh:
        for line in fh:
            line = line.split("#")[0].split()
            if not line:
                continue
            if line[0] == "topo":
                bar = line.index("|")
                nums = list(map(int, line[1:bar]))
                topo = (nums[0], nums[1], nums[2:], list(map(int, line[bar + 1:])))
                C = [[0] * len(topo[2]) for _ in topo[2]]
            elif line[0] == "C":
                u, v, b = map(int, line[1:])
                C[u][v] = b
            elif line[0] == "stage":
                s, k, u, v, b = map(int, line[1:])
                stages.setdefault(s, []).append((k, u, v, b))
            elif line[0] == "tau":
                s, L, B = map(int, line[1:])
                taus[s] = (L, B)
    return C, topo, stages, taus


def test_golden_hand_worked_decomposition():
    C, (bnv, brd, node, peer), stages, taus = _read_golden("schedule_g4_two_nodes.txt")
    got = cs.decompose(C, node, peer, bnv, brd)
    assert len(got) == len(stages)
    for s, st in enumerate(got):
        assert st["entries"] == sorted(stages[s])
        assert st["tau"] == taus[s]
    assert cs.total_time(got) == 5.0


@pytest.mark.parametrize("case", range(len(CASES)))
def test_completeness_eq7(case):
    t, C = CASES[case]
    T = cs.traffic_matrix(C, t.node(), t.peer())
    st = cs.decompose(C, t.node(), t.peer(), t.bw_scaleup, t.bw_rdma)
    total = [[0] * t.G for _ in range(t.G)]
    for M in cs.stage_matrices(st, t.G):
        for u, v in itertools.product(range(t.G), range(t.G)):
            total[u][v] += M[u][v]
    assert total == T
    # every entry is positive and on an edge of the right domain
    for s in st:
        for k, u, v, b in s["entries"]:
            assert b > 0 and u != v
            assert (k == cs.RDMA) == _rdma(t, u, v)
            if k == cs.FWD:
                assert t.peer()[u] == v or t.peer()[v] == u


@pytest.mark.parametrize("case", range(len(CASES)))
def test_degree_constraint_eq8(case):
    t, C = CASES[case]
    st = cs.decompose(C, t.node(), t.peer(), t.bw_scaleup, t.bw_rdma)
    for s in st:
        rd = [(u, v) for k, u, v, _ in s["entries"] if k == cs.RDMA]
        assert len({u for u, _ in rd}) == len(rd)
        assert len({v for _, v in rd}) == len(rd)


@pytest.mark.parametrize("case", range(len(CASES)))
def test_forwarding_and_bvn_step(case):
    """Each RDMA stage moves one amount x on every matched flow (reading (b));
    its forwarding entries are exactly x per matched flow on (u, peer u) and
    (peer v, v) (Eq. 2); some flow empties every stage, so there are at most
    as many RDMA stages as RDMA flows, and at least as many as the largest
    RDMA degree of a GPU (a stage carries one flow per sender and receiver)."""
    t, C = CASES[case]
    node, peer = t.node(), t.peer()
    st = cs.decompose(C, node, peer, t.bw_scaleup, t.bw_rdma)
    n_rdma = 0
    for s in st:
        rd = [(u, v, b) for k, u, v, b in s["entries"] if k == cs.RDMA]
        if not rd:
            continue
        n_rdma += 1
        xs = {b for _, _, b in rd}
        assert len(xs) == 1
        x = xs.pop()
        want = {}
        for u, v, _ in rd:
            if peer[u] >= 0:
                want[(u, peer[u])] = want.get((u, peer[u]), 0) + x
            if peer[v] >= 0:
                want[(peer[v], v)] = want.get((peer[v], v), 0) + x
        got = {(u, v): b for k, u, v, b in s["entries"] if k == cs.FWD}
        assert got == want
    flows = [(u, v) for u in range(t.G) for v in range(t.G) if _rdma(t, u, v) and C[u][v] > 0]
    assert n_rdma <= len(flows)
    deg = max([sum(1 for f in flows if f[0] == g) for g in range(t.G)] +
              [sum(1 for f in flows if f[1] == g) for g in range(t.G)] + [0])
    assert n_rdma >= deg
    # RDMA stages come first; the native tail follows (reading (e))
    kinds = [any(k == cs.RDMA for k, *_ in s["entries"]) for s in st]
    assert kinds == sorted(kinds, reverse=True)


@pytest.mark.parametrize("case", range(len(CASES)))
def test_stage_time_eq9_eq10(case):
    """tau^s bounds every entry of its stage (Eq. 9, 10); summed, the stage
    times bound every entry of T and every GPU's total RDMA bytes, since a
    GPU sends and receives at most one RDMA flow per stage (Eq. 8)."""
    t, C = CASES[case]
    node, peer = t.node(), t.peer()
    T = cs.traffic_matrix(C, node, peer)
    st = cs.decompose(C, node, peer, t.bw_scaleup, t.bw_rdma)
    from fractions import Fraction as Fr
    total = Fr(0)
    for s, M in zip(st, cs.stage_matrices(st, t.G)):
        L, B = s["tau"]
        tau = Fr(L, B)
        assert B in (t.bw_scaleup, t.bw_rdma)
        hit = False
        for u, v in itertools.product(range(t.G), range(t.G)):
            bw = t.bw_rdma if _rdma(t, u, v) else t.bw_scaleup
            assert Fr(M[u][v], bw) <= tau
            hit |= Fr(M[u][v], bw) == tau
        assert hit  # the slowest domain's largest entry sets the time
        total += tau
    for u, v in itertools.product(range(t.G), range(t.G)):
        bw = t.bw_rdma if _rdma(t, u, v) else t.bw_scaleup
        assert Fr(T[u][v], bw) <= total
    for g in range(t.G):
        out = sum(C[g][v] for v in range(t.G) if _rdma(t, g, v))
        inc = sum(C[u][g] for u in range(t.G) if _rdma(t, u, g))
        assert Fr(max(out, inc), t.bw_rdma) <= total
    assert cs.total_time(st) == pytest.approx(float(total))


@pytest.mark.parametrize("case", range(len(CASES)))
def test_slack_fill_keeps_rdma_time(case):
    """Native traffic packed into an RDMA stage never makes the stage longer
    than its RDMA transfer or its forwarding copies would (reading (d))."""
    t, C = CASES[case]
    st = cs.decompose(C, t.node(), t.peer(), t.bw_scaleup, t.bw_rdma)
    for s in st:
        rd = [b for k, _, _, b in s["entries"] if k == cs.RDMA]
        if not rd:
            continue
        fwd = {}
        for k, u, v, b in s["entries"]:
            if k == cs.FWD:
                fwd[(u, v)] = fwd.get((u, v), 0) + b
        without_native = {(k, u, v): b for k, u, v, b in s["entries"] if k != cs.NATIVE}
        assert s["tau"] == cs.stage_time(without_native, t.bw_scaleup, t.bw_rdma) or \
            s["tau"][0] * t.bw_rdma <= rd[0] * t.bw_scaleup


def test_native_only_reduces_to_birkhoff_von_neumann():
    """With one node there is no RDMA domain and the decomposition is the
    matching peel of Birkhoff-von Neumann: a matrix a*P1 + b*P2 (P1, P2
    permutation matrices without common or diagonal entries, a > b > 0)
    comes apart into exactly those two stages."""
    G = 6
    P1 = [(u, (u + 1) % G) for u in range(G)]
    P2 = [(u, (u + 3) % G) for u in range(G)]
    a, b = 700, 300
    C = [[0] * G for _ in range(G)]
    for u, v in P1:
        C[u][v] += a
    for u, v in P2:
        C[u][v] += b
    st = cs.decompose(C, [0] * G, [-1] * G, 10, 1)
    assert [s["entries"] for s in st] == [sorted((cs.NATIVE, u, v, a) for u, v in P1),
                                           sorted((cs.NATIVE, u, v, b) for u, v in P2)]
    assert [s["tau"] for s in st] == [(a, 10), (b, 10)]


def test_rdma_permutation_lasts_its_largest_flow():
    """A pure inter-node permutation without forwarding is contention-free:
    every stage carries every flow that still has bytes left, the BvN step
    empties the smallest, and the stages add up to the largest flow's time."""
    t = W.Topology("2x3", 2, 3, 9, 2, paired=False)
    C = [[0] * 6 for _ in range(6)]
    for u, s in zip(range(3), (5, 9, 4)):
        C[u][u + 3] = s
        C[u + 3][u] = s + 1
    st = cs.decompose(C, t.node(), t.peer(), t.bw_scaleup, t.bw_rdma)
    left = {(u, v): C[u][v] for u in range(6) for v in range(6) if C[u][v]}
    for s in st:
        live = sorted(p for p, r in left.items() if r > 0)
        assert sorted((u, v) for _, u, v, _ in s["entries"]) == live
        x = min(left[p] for p in live)
        assert all(b == x for *_, b in s["entries"])
        for p in live:
            left[p] -= x
    assert not any(left.values())
    assert [s["tau"] for s in st] == [(4, 2), (1, 2), (1, 2), (3, 2), (1, 2)]
    assert cs.total_time(st) == max(map(max, C)) / t.bw_rdma


def test_greedy_matching_is_maximal_brute_force():
    """Reading (a) on every 0/1 pattern of a 3 x 3 bipartite block: the
    matching is valid and no remaining edge could join it."""
    for bits in range(1 << 9):
        resid = {(u, 3 + v): (bits >> (3 * u + v) & 1) * (1 + u + 2 * v)
                 for u in range(3) for v in range(3)}
        m = cs.greedy_matching(resid)
        assert len({u for u, _ in m}) == len(m) == len({v for _, v in m})
        su, sv = {u for u, _ in m}, {v for _, v in m}
        for (u, v), r in resid.items():
            if r > 0:
                assert (u, v) in m or u in su or v in sv
        # first pick is a largest entry (decreasing residual)
        if m:
            assert resid[m[0]] == max(resid.values())


def test_empty_and_degenerate():
    t = W.FIG6_TOPOLOGY
    Z = [[0] * 4 for _ in range(4)]
    assert cs.decompose(Z, t.node(), t.peer(), 3, 1) == []
    assert cs.traffic_matrix(Z, t.node(), t.peer()) == Z
    # diagonal entries are not traffic
    D = [[7 if u == v else 0 for v in range(4)] for u in range(4)]
    assert cs.decompose(D, t.node(), t.peer(), 3, 1) == []


def test_moe_workload_schedule_properties():
    w = W.SCHED_MOE_2X8
    t = w.topology
    C = W.moe_traffic(w)
    row = w.hidden * 2
    for u in range(t.G):
        assert C[u][u] == 0 and sum(C[u]) <= w.tokens * w.topk * row
        assert all(b % row == 0 for b in C[u])
    st = cs.decompose(C, t.node(), t.peer(), t.bw_scaleup, t.bw_rdma)
    T = cs.traffic_matrix(C, t.node(), t.peer())
    total = [[0] * t.G for _ in range(t.G)]
    for M in cs.stage_matrices(st, t.G):
        for u, v in itertools.product(range(t.G), range(t.G)):
            total[u][v] += M[u][v]
    assert total == T
