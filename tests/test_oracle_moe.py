"""Pins of the CPU oracle's expert-parallel dispatch and combine.  No GPU."""
import os

import numpy as np
import pytest

import oracle
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load_golden():
    g = {}
    for line in open(os.path.join(GOLDEN, "moe_tiny_r2_t4_e4_k2.txt")):
        line = line.split("#")[0].split()
        if line:
            g.setdefault(line[0], []).append(line[1:])
    return g


def _pairs(vals):
    return [tuple(int(x) for x in v.split(":")) for v in vals]


def test_golden_tiny_dispatch():
    g = _load_golden()
    R, T, E, K = 2, 4, 4, 2
    logits = [np.zeros((T, E), np.float32) for _ in range(R)]
    for r, t, *v in g["logits"]:
        logits[int(r)][int(t)] = np.array(v, np.float32)
    topks = [oracle.moe_topk(l, K) for l in logits]
    for r, t, *v in g["topk"]:
        assert topks[int(r)][int(t)].tolist() == [int(x) for x in v]
    # activations whose row (r, t) encodes r and t
    xs = [np.array([[r * 100 + t] * 3 for t in range(T)], np.int32) for r in range(R)]
    plan = oracle.moe_dispatch(xs, topks, E)
    for r, *v in g["send_tok"]:
        assert plan["src_tok"][int(r)].tolist() == [int(x) for x in v]
    for r, t, *v in g["slot"]:
        assert plan["slot"][int(r)][int(t)].tolist() == [int(x) for x in v]
    for r, *v in g["counts"]:
        assert plan["counts"][int(r)].tolist() == [int(x) for x in v]
    for r, *v in g["ecnt"]:
        assert plan["ecnt"][int(r)].tolist() == [int(x) for x in v]
    for d, *v in g["recv"]:
        assert [(x // 100, x % 100) for x in plan["recv"][int(d)][:, 0]] == _pairs(v)
    for d, *v in g["unpack"]:
        assert plan["unpack"][int(d)].tolist() == [int(x) for x in v]
    for d, *v in g["exp"]:
        assert [(x // 100, x % 100) for x in plan["exp"][int(d)][:, 0]] == _pairs(v)
    out = oracle.moe_combine(plan["exp"], plan)
    for r in range(R):
        for t in range(T):
            for k in range(K):
                assert out[r][t, k].tolist() == xs[r][t].tolist()


@pytest.mark.parametrize("T,E,K", [(64, 16, 4), (300, 64, 6), (5, 8, 8), (17, 8, 1)])
def test_topk_matches_stable_argsort(T, E, K):
    """Top-K by decreasing logit with ties to the lower id is the first K of
    numpy's stable argsort of -logits (a library routine).  Ties are forced
    by quantising the logits."""
    rng = np.random.default_rng(T + E)
    logits = np.round(rng.normal(0, 1, (T, E)) * 2) / 2
    logits = logits.astype(np.float32)
    ref = np.argsort(-logits, axis=1, kind="stable")[:, :K].astype(np.int32)
    np.testing.assert_array_equal(oracle.moe_topk(logits, K), ref)


@pytest.mark.parametrize("R,T,E,K", [(2, 50, 8, 2), (4, 257, 16, 3), (8, 128, 64, 6)])
def test_dispatch_properties_and_round_trip(R, T, E, K):
    """Every (token, choice) is packed exactly once; the rows that reach
    expert e are exactly the tokens that chose e, ordered by (source, token);
    counts are conserved; combine returns every token to every slot."""
    w = workloads.MOE_DISPATCH_BF16
    _, logits = workloads.moe_inputs(w, tokens=T, R=R)
    logits = [l[:, :E].copy() for l in logits]
    topks = [oracle.moe_topk(l, K) for l in logits]
    xs = [np.array([[r * 100000 + t] * 2 for t in range(T)], np.int32) for r in range(R)]
    plan = oracle.moe_dispatch(xs, topks, E)
    eloc = E // R
    assert plan["counts"].sum() == R * T * K
    np.testing.assert_array_equal(plan["counts"].sum(axis=1), np.full(R, T * K))
    for r in range(R):
        slot = plan["slot"][r]
        assert sorted(slot.ravel().tolist()) == list(range(T * K))
        np.testing.assert_array_equal(plan["src_tok"][r][slot], np.repeat(np.arange(T), K).reshape(T, K))
    for d in range(R):
        rows = plan["exp"][d][:, 0].tolist()
        expect = []
        for l in range(eloc):
            e = d * eloc + l
            for r in range(R):
                expect += [r * 100000 + t for t in range(T) if e in topks[r][t]]
        assert rows == expect
    out = oracle.moe_combine(plan["exp"], plan)
    for r in range(R):
        np.testing.assert_array_equal(out[r][:, :, 0], np.repeat(np.arange(T)[:, None] + r * 100000, K, 1))


def test_moe_workload_routing_shape():
    w = workloads.MOE_DISPATCH_BF16
    xs, logits = workloads.moe_inputs(w, tokens=16, R=2)
    assert xs[0].shape == (16, 2048) and xs[0].dtype == np.uint16
    assert logits[0].shape == (16, 64) and logits[0].dtype == np.float32
    tk = oracle.moe_topk(logits[0], w.topk)
    assert tk.shape == (16, 6)
    assert all(len(set(row)) == 6 for row in tk.tolist())
