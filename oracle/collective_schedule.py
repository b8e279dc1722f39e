"""Oracle for the collective scheduler's stage decomposition.

TEST INFRASTRUCTURE ONLY: imported by tests/, the package smoke check and the
benchmark's CPU baseline, never by the library or its binding.

Plain Python written from "HOCCL: Offloading Collective Communication from
GPU Cores to Accelerate Distributed Training", §3.4 Collective Scheduler
(Figure 6, Eq. 2-11, Algorithm 1), in the paper's notation:

  C        origin traffic matrix: C[u][v] = bytes of the logical flow g_u -> g_v
  node[u]  the scale-up domain (node) of GPU u; flows between nodes are RDMA
  peer[u]  ū, the symmetric peer of u; an inter-node flow u -> v is realised as
           a sender-side forwarding copy on (u, ū), the RDMA transfer, and a
           receiver-side forwarding copy on (v̄, v) (Eq. 2).  -1: u needs no
           forwarding copy.
  A_u, B_v sums of u's outgoing and v's incoming inter-node flows (Eq. 3)
  T        HOCCL traffic matrix: T[u][ū] = C[u][ū] + A_u + B_ū on the edge to
           the symmetric peer, T = C elsewhere (Eq. 4, 5)
  T^s      stage matrices: sum_s T^s = T element-wise (Eq. 7); at most one
           outgoing and one incoming RDMA entry per GPU per stage (Eq. 8)
  L^s_d    the largest entry of domain d in stage s (Eq. 9)
  tau^s    max_d L^s_d / B_d (Eq. 10); the schedule's cost is sum_s tau^s (Eq. 11)

Where Algorithm 1 leaves a step open, these readings are taken:
  (a) a matching (of the native components, and the contention-free RDMA
      set of each stage) is built greedily: entries with traffic
      left, by decreasing residual, ties by (u, v); an entry joins when its
      sender has no outgoing and its receiver no incoming entry yet.  Native
      scale-up traffic is decomposed node by node.
  (b) the largest portion a stage can remove is the smallest residual over
      the matching, the Birkhoff-von Neumann coefficient: every matched entry
      moves that much, so at least one of them empties.
  (c) forwarding copies: a moved portion x of u -> v adds x on (u, ū)
      and x on (v̄, v).
  (d) scale-up slack: with the stage lasting at least x / B_rdma,
      every scale-up edge may carry cap = max(floor(x * B_nv / B_rdma), the
      largest forwarding load of the stage); native components, node by node
      and in decomposition order, each move min(what is left, the least room
      over its edges) on all their edges.
  (e) native traffic left after the RDMA traffic is exhausted forms further
      stages; stage i of that tail holds the first remaining component of
      every node.
Every quantity is an integer (bytes; bandwidths in bytes per time unit), and
tau is kept as an exact ratio, so two implementations agree bit for bit.
"""
from __future__ import annotations

RDMA, FWD, NATIVE = 0, 1, 2  # kinds of stage entries


def traffic_matrix(C, node, peer):
    """Eq. 2-5: the HOCCL traffic matrix T from the origin matrix C."""
    G = len(C)
    A = [0] * G  # Eq. 3, sender side
    B = [0] * G  # Eq. 3, receiver side
    for u in range(G):
        for v in range(G):
            if u != v and node[u] != node[v]:
                if peer[u] >= 0:
                    A[u] += C[u][v]
                if peer[v] >= 0:
                    B[v] += C[u][v]
    T = [[C[u][v] if u != v else 0 for v in range(G)] for u in range(G)]
    for u in range(G):
        if peer[u] >= 0:
            T[u][peer[u]] += A[u] + B[peer[u]]  # Eq. 4
    return T


def greedy_matching(resid):
    """Reading (a): resid maps (u, v) -> bytes left; returns matched pairs."""
    order = sorted((-r, u, v) for (u, v), r in resid.items() if r > 0)
    senders, receivers, match = set(), set(), []
    for _, u, v in order:
        if u not in senders and v not in receivers:
            match.append((u, v))
            senders.add(u)
            receivers.add(v)
    return match


def native_components(C, node):
    """Algorithm 1, first step: per node, matchings peeled off the native traffic.
    Returns {node: [[pairs, bytes], ...]} in decomposition order."""
    G = len(C)
    comps = {}
    for n in sorted(set(node)):
        resid = {(u, v): C[u][v] for u in range(G) for v in range(G)
                 if u != v and node[u] == n and node[v] == n and C[u][v] > 0}
        lst = []
        while any(resid.values()):
            m = greedy_matching(resid)
            w = min(resid[p] for p in m)
            for p in m:
                resid[p] -= w
            lst.append([m, w])
        comps[n] = lst
    return comps


def _add(stage, kind, u, v, amount):
    stage[(kind, u, v)] = stage.get((kind, u, v), 0) + amount


def decompose(C, node, peer, bw_nv, bw_rdma):
    """Algorithm 1.  Returns a list of stages, each {"entries": sorted list of
    (kind, u, v, bytes), "tau": (bytes, bandwidth)} where tau^s equals
    bytes / bandwidth of the stage's slowest domain (Eq. 9, 10)."""
    G = len(C)
    comps = native_components(C, node)
    resid = {(u, v): C[u][v] for u in range(G) for v in range(G)
             if node[u] != node[v] and C[u][v] > 0}          # RDMA part of the residual
    stages = []
    while any(resid.values()):
        st = {}
        m = greedy_matching(resid)                           # reading (a)
        x = min(resid[p] for p in m)                         # reading (b)
        load = {}
        for u, v in m:
            resid[(u, v)] -= x
            _add(st, RDMA, u, v, x)
        for u, v in m:                                       # reading (c)
            if peer[u] >= 0:
                _add(st, FWD, u, peer[u], x)
                load[(u, peer[u])] = load.get((u, peer[u]), 0) + x
            if peer[v] >= 0:
                _add(st, FWD, peer[v], v, x)
                load[(peer[v], v)] = load.get((peer[v], v), 0) + x
        cap = max(x * bw_nv // bw_rdma, max(load.values(), default=0))
        for n in sorted(comps):                              # reading (d)
            for comp in comps[n]:
                pairs, left = comp
                if left == 0:
                    continue
                amount = min([left] + [cap - load.get(p, 0) for p in pairs])
                if amount > 0:
                    for u, v in pairs:
                        _add(st, NATIVE, u, v, amount)
                        load[(u, v)] = load.get((u, v), 0) + amount
                    comp[1] -= amount
        stages.append(st)
    while True:                                              # reading (e)
        st = {}
        for n in sorted(comps):
            for comp in comps[n]:
                if comp[1] > 0:
                    for u, v in comp[0]:
                        _add(st, NATIVE, u, v, comp[1])
                    comp[1] = 0
                    break
        if not st:
            break
        stages.append(st)
    return [{"entries": sorted((k, u, v, b) for (k, u, v), b in st.items()),
             "tau": stage_time(st, bw_nv, bw_rdma)} for st in stages]


def stage_time(st, bw_nv, bw_rdma):
    """Eq. 9, 10 for one stage given as {(kind, u, v): bytes}: the slowest
    domain's (L, B).  Scale-up cells sum their native and forwarding bytes;
    every scale-up domain has bandwidth bw_nv, so the largest such cell over
    all nodes decides."""
    rd = max((b for (k, u, v), b in st.items() if k == RDMA), default=0)
    cells = {}
    for (k, u, v), b in st.items():
        if k != RDMA:
            cells[(u, v)] = cells.get((u, v), 0) + b
    nv = max(cells.values(), default=0)
    return (rd, bw_rdma) if rd * bw_nv >= nv * bw_rdma else (nv, bw_nv)


def stage_matrices(stages, G):
    """T^s as G x G integer matrices."""
    out = []
    for st in stages:
        M = [[0] * G for _ in range(G)]
        for _, u, v, b in st["entries"]:
            M[u][v] += b
        out.append(M)
    return out


def total_time(stages):
    """Eq. 11: sum over stages of tau^s, as a float."""
    return sum(b / bw for b, bw in (s["tau"] for s in stages))
