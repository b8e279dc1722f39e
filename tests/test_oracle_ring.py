"""Pins of the CPU oracle's ring reduce-scatter / all-gather.

Each test checks the oracle against something that does not come from the
oracle: exact integer sums, IEEE rounding facts, rounding-error bounds,
library routines (numpy float32 add, torch's bf16 cast and bf16 add) and a
hand-worked fixture.  No GPU is needed.
"""
import os

import numpy as np
import pytest
import torch

import oracle
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ------------------------------------------------------------ partition
@pytest.mark.parametrize("n,R", [(0, 1), (1, 1), (1, 4), (7, 3), (12, 3), (1000, 7),
                                 (1 << 20, 4), (26214400, 8), (8388608, 32), (33, 64), (5, 64)])
@pytest.mark.parametrize("vec", [4, 8])
def test_partition_covers_range_aligned(n, R, vec):
    """Chunks tile [0, n) in order, without gaps or overlap, start on a
    16-byte boundary, and the slices of each chunk tile the chunk."""
    pos = 0
    for c in range(R):
        lo, hi = oracle.chunk_bounds(n, R, vec, c)
        assert lo == pos and lo <= hi <= n
        assert lo % vec == 0 or lo == n
        pos = hi
        for S in (1, 2, 3, 4, 7):
            spos = lo
            for s in range(S):
                slo, shi = oracle.slice_bounds(lo, hi, S, vec, s)
                assert slo == spos and slo <= shi <= hi
                assert (slo - lo) % vec == 0 or slo == hi
                spos = shi
            assert spos == hi
    assert pos == n
    # every chunk but the trailing ones has the full aligned length
    full = -(-(-(-n // R)) // vec) * vec
    lens = [oracle.chunk_bounds(n, R, vec, c)[1] - oracle.chunk_bounds(n, R, vec, c)[0]
            for c in range(R)]
    assert all(L <= full for L in lens)
    assert lens == sorted(lens, reverse=True)


# ----------------------------------------------------- exact integer sums
@pytest.mark.parametrize("R,n,S", [(2, 40, 1), (3, 12, 2), (5, 1001, 3), (8, 4096, 4),
                                   (17, 333, 2), (32, 2048, 4), (64, 777, 1)])
def test_fp32_allreduce_equals_exact_sum_on_integers(R, n, S):
    """Integers with |x| <= 2^10 and R <= 64 keep every partial below 2^24,
    so each fp32 add is exact and the ring must give the exact sum."""
    xs = workloads.integer_buffers(R, n, "f32", seed=R * 1000 + n, bound=1 << 10)
    exact = np.sum(np.stack(xs).astype(np.int64), axis=0)
    out = oracle.ring_allreduce(xs, S=S)
    for q in range(R):
        np.testing.assert_array_equal(out[q].astype(np.int64), exact)


@pytest.mark.parametrize("R,n,S", [(2, 24, 1), (3, 100, 2), (8, 4097, 4)])
@pytest.mark.parametrize("acc", ["per_hop", "fp32_partials"])
def test_bf16_allreduce_equals_exact_sum_on_small_integers(R, n, S, acc):
    """|x| <= 16 and R <= 8 keep every partial within +-128, which bf16's
    8-bit significand holds exactly, so both bf16 modes give the exact sum."""
    xs = workloads.integer_buffers(R, n, "bf16", seed=R * 7 + n, bound=16)
    vals = [oracle.bf16_to_f32(x).astype(np.int64) for x in xs]
    exact = np.sum(np.stack(vals), axis=0)
    out = oracle.ring_allreduce(xs, S=S, bf16_acc=acc)
    for q in range(R):
        np.testing.assert_array_equal(oracle.bf16_to_f32(out[q]).astype(np.int64), exact)


# ------------------------------------------------------- special cases
def test_single_rank_is_identity():
    for dt in ("f32", "bf16"):
        xs = workloads.random_buffers(1, 1003, dt, seed=3)
        out = oracle.ring_allreduce(xs, S=3)
        np.testing.assert_array_equal(out[0], xs[0])


def test_two_ranks_fp32_is_one_ieee_add():
    """R = 2: every element is a single float32 add, which numpy performs
    in IEEE binary32 with round-to-nearest-even."""
    a, b = workloads.random_buffers(2, 10007, "f32", seed=11)
    out = oracle.ring_allreduce([a, b], S=2)
    ref = (a + b).astype(np.float32)
    for q in range(2):
        assert out[q].tobytes() == ref.tobytes()


def test_two_ranks_bf16_is_one_torch_bf16_add():
    """R = 2: one bf16 hop; torch's CPU bf16 add widens to fp32, adds and
    rounds to nearest even -- an independent implementation of the hop."""
    a, b = workloads.random_buffers(2, 10007, "bf16", seed=12, dist="normal", scale=1e-3)
    ta = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16)
    tb = torch.from_numpy(b.view(np.int16)).view(torch.bfloat16)
    ref = (ta + tb).view(torch.int16).numpy().view(np.uint16)
    for acc in ("per_hop", "fp32_partials"):
        out = oracle.ring_allreduce([a, b], S=1, bf16_acc=acc)
        np.testing.assert_array_equal(out[0], ref)
        np.testing.assert_array_equal(out[1], ref)


def test_zero_length_and_empty_chunks():
    """n < R*V leaves trailing chunks empty; n = 0 is a no-op."""
    xs = workloads.integer_buffers(5, 3, "f32", seed=1, bound=100)
    exact = np.sum(np.stack(xs), axis=0)
    out = oracle.ring_allreduce(xs)
    for q in range(5):
        np.testing.assert_array_equal(out[q], exact)
    out = oracle.ring_allreduce([np.zeros(0, np.float32)] * 3)
    assert all(o.size == 0 for o in out)


# --------------------------------------------------- hand-worked fixture
def _golden_ring():
    lines = [l.split("#")[0].strip() for l in open(os.path.join(GOLDEN, "ring_r3_hops.txt"))]
    states, finals = {}, {}
    for l in lines:
        if not l:
            continue
        tag, rest = l.split(None, 1)
        if tag.startswith("final_"):
            finals[tag] = float(rest)
        else:
            states[tag] = [[float(v) for v in grp.split()] for grp in rest.split("|")]
    return states, finals


def test_golden_ring_r3_hops_and_order():
    states, finals = _golden_ring()
    R, n, u = 3, 12, np.float32(2.0 ** -24)
    xs = [np.zeros(n, np.float32) for _ in range(R)]
    for q in range(R):
        for c in range(R):
            base = 4 * c
            xs[q][base + 3] = (q + 1) * (c + 1)
            # order-sensitive elements (see the fixture's comments)
            xs[q][base + 0] = 1.0 if q == c else u
            xs[q][base + 1] = 1.0 if q == (c + 1) % R else u
            xs[q][base + 2] = 1.0 if q == (c + 2) % R else u
    bufs = [x.copy() for x in xs]

    def elem3(b):
        return [[float(b[q][4 * c + 3]) for c in range(R)] for q in range(R)]

    assert elem3(bufs) == states["init"]
    for k in range(R - 1):
        oracle.ring_step(bufs, "rs", k)
        assert elem3(bufs) == states[f"rs{k}"], f"after reduce-scatter hop {k}"
    for k in range(R - 1):
        oracle.ring_step(bufs, "ag", k)
        assert elem3(bufs) == states[f"ag{k}"], f"after all-gather hop {k}"
    for q in range(R):
        for c in range(R):
            assert bufs[q][4 * c + 0] == np.float32(finals["final_e0"])
            assert bufs[q][4 * c + 1] == np.float32(finals["final_e1"])
            assert bufs[q][4 * c + 2] == np.float32(finals["final_e2"])
    assert np.float32(finals["final_e0"]) == np.float32(1.0) + np.float32(2.0 ** -23)
    # the whole-collective entry point and the closed form agree with the hops
    full = oracle.ring_allreduce(xs)
    for q in range(R):
        np.testing.assert_array_equal(full[q], bufs[q])
    np.testing.assert_array_equal(oracle.fold(xs), bufs[0])


# ------------------------------------------------------- error bounds
def _gamma(m, u):
    return m * u / (1 - m * u)


@pytest.mark.parametrize("R", [2, 4, 8, 32])
def test_fp32_within_recursive_summation_bound(R):
    """|ring - exact| <= gamma_{R-1} * sum|x| with u = 2^-24 (recursive
    summation bound, Higham, Accuracy and Stability, Sec. 4.2); the exact
    sum of float32 values is exact in float64 for these magnitudes."""
    xs = workloads.random_buffers(R, 20011, "f32", seed=100 + R)
    out = oracle.ring_allreduce(xs, S=2)[0].astype(np.float64)
    X = np.stack(xs).astype(np.float64)
    exact = X.sum(axis=0)
    bound = _gamma(R - 1, 2.0 ** -24) * np.abs(X).sum(axis=0)
    assert np.all(np.abs(out - exact) <= bound)


@pytest.mark.parametrize("R", [2, 4, 8])
def test_bf16_per_hop_within_bound_and_tolerance(R):
    """Each bf16 hop returns the correctly rounded bf16 sum (unit roundoff
    2^-8), so the recursive summation bound holds with u = 2^-8; and the
    normalised max error stays under the 1e-2 accuracy bar."""
    xs = workloads.random_buffers(R, 50021, "bf16", seed=200 + R, dist="normal", scale=1e-3)
    out = oracle.bf16_to_f32(oracle.ring_allreduce(xs, S=4)[0]).astype(np.float64)
    X = np.stack([oracle.bf16_to_f32(x) for x in xs]).astype(np.float64)
    exact = X.sum(axis=0)
    bound = _gamma(R - 1, 2.0 ** -8) * np.abs(X).sum(axis=0)
    assert np.all(np.abs(out - exact) <= bound)
    assert np.max(np.abs(out - exact)) <= 1e-2 * np.max(np.abs(exact))


@pytest.mark.parametrize("R", [3, 8])
def test_bf16_fp32_partials_within_bound(R):
    """fp32 partials: the fp32 fold error plus one final bf16 rounding."""
    xs = workloads.random_buffers(R, 30011, "bf16", seed=300 + R, dist="normal", scale=1.0)
    out = oracle.bf16_to_f32(oracle.ring_allreduce(xs, S=2, bf16_acc="fp32_partials")[0])
    X = np.stack([oracle.bf16_to_f32(x) for x in xs]).astype(np.float64)
    exact = X.sum(axis=0)
    fold_err = _gamma(R - 1, 2.0 ** -24) * np.abs(X).sum(axis=0)
    bound = fold_err + 2.0 ** -8 * (np.abs(exact) + fold_err)
    assert np.all(np.abs(out.astype(np.float64) - exact) <= bound)


# ------------------------------------------------------------ invariants
@pytest.mark.parametrize("dt,acc", [("f32", "per_hop"), ("bf16", "per_hop"), ("bf16", "fp32_partials")])
@pytest.mark.parametrize("R,n", [(3, 1001), (5, 4099), (8, 65537)])
def test_invariants(dt, acc, R, n):
    """All ranks identical; the result does not depend on S; the hop-by-hop
    simulation equals the closed-form fold (the partial starts at c+1 and
    the owner adds last); reduce-scatter leaves chunk c reduced on rank c;
    all-gather is a pure permutation of chunk c of rank c."""
    xs = workloads.random_buffers(R, n, dt, seed=R * n, dist="normal", scale=1.0)
    ref = oracle.ring_allreduce(xs, S=1, bf16_acc=acc)
    for q in range(1, R):
        assert ref[q].tobytes() == ref[0].tobytes()
    for S in (2, 3, 7):
        out = oracle.ring_allreduce(xs, S=S, bf16_acc=acc)
        assert out[0].tobytes() == ref[0].tobytes()
    assert oracle.fold(xs, bf16_acc=acc).tobytes() == ref[0].tobytes()
    idx = np.random.default_rng(R).integers(0, n, 257)
    np.testing.assert_array_equal(oracle.fold_at(xs, idx, bf16_acc=acc), ref[0][idx])
    vec = 4 if dt == "f32" else 8
    rs = oracle.ring_reduce_scatter(xs, S=2, bf16_acc=acc)
    for c in range(R):
        lo, hi = oracle.chunk_bounds(n, R, vec, c)
        np.testing.assert_array_equal(rs[c][lo:hi], ref[0][lo:hi])
    # all-gather on arbitrary (unreduced) inputs: rank q ends holding chunk c
    # of rank c for every c, bit for bit
    ag = oracle.ring_all_gather(xs, S=3)
    expect = np.concatenate([xs[c][slice(*oracle.chunk_bounds(n, R, vec, c))] for c in range(R)])
    for q in range(R):
        np.testing.assert_array_equal(ag[q], expect)
    both = oracle.ring_all_gather(rs, S=1)
    for q in range(R):
        np.testing.assert_array_equal(both[q], ref[q])


# ------------------------------------------------------------------ bf16
def test_bf16_rounding_matches_torch_cast():
    """The oracle's float32 -> bf16 rounding equals torch's cast (a library
    routine, round to nearest even) on a sweep of bit patterns: random
    words, exact ties, tie +- 1 ulp, denormals, powers of two, extremes."""
    rng = np.random.default_rng(5)
    words = [rng.integers(0, 2 ** 32, 200000, dtype=np.uint64).astype(np.uint32)]
    hi = rng.integers(0, 2 ** 16, 20000, dtype=np.uint64).astype(np.uint32) << 16
    for low in (0x8000, 0x7FFF, 0x8001, 0x0000, 0xFFFF, 0x0001):
        words.append(hi | np.uint32(low))
    words.append(np.arange(0, 1 << 16, dtype=np.uint32))            # denormals
    words.append((np.arange(0, 255, dtype=np.uint32) << 23))         # powers of 2
    words.append(np.array([0x7F7FFFFF, 0xFF7FFFFF, 0x7F800000, 0xFF800000,
                           0x80000000, 0x7F7F8000, 0x00008000, 0x80018000], np.uint32))
    w = np.concatenate(words)
    f = w.view(np.float32)
    keep = ~np.isnan(f)
    f = f[keep]
    got = oracle.f32_to_bf16(f)
    ref = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(got, ref)
    # widening is exact: bf16 -> f32 -> bf16 is the identity
    np.testing.assert_array_equal(oracle.f32_to_bf16(oracle.bf16_to_f32(ref)), ref)


@pytest.mark.parametrize("dt,acc", [("f32", "per_hop"), ("bf16", "per_hop"), ("bf16", "fp32_partials")])
@pytest.mark.parametrize("R,n,S", [(1, 50, 1), (2, 1001, 2), (5, 40013, 3), (8, 65536 + 9, 1)])
def test_range_entry_point_equals_the_unsplit_oracle(dt, acc, R, n, S):
    """Running the all-reduce over disjoint element windows that cover the
    buffers -- at cut points that fall inside chunks, slices and 16-byte
    vectors, with empty windows among them, sequentially and on threads --
    leaves every buffer bit for bit as the unsplit oracle does."""
    if dt == "f32" and acc != "per_hop":
        pytest.skip("fp32 has one accumulation mode")
    xs = workloads.random_buffers(R, n, dt, seed=R * 13 + n, dist="normal", scale=1.0)
    ref = oracle.ring_allreduce(xs, S=S, bf16_acc=acc)
    rng = np.random.default_rng(n)
    cuts = np.unique(np.concatenate([[0, n, n // 3, n // 3], rng.integers(0, n + 1, 6)]))
    cuts = np.concatenate([cuts, [n]])  # an empty last window
    bufs = [x.copy() for x in xs]
    part = [np.zeros(n, np.float32) for _ in range(R)] if acc == "fp32_partials" else None
    order = rng.permutation(len(cuts) - 1)
    for i in order:  # windows in a shuffled order
        oracle.ring_allreduce_range(bufs, int(cuts[i]), int(cuts[i + 1]), S, acc, part)
    for q in range(R):
        assert bufs[q].tobytes() == ref[q].tobytes(), f"rank {q}"
    got = oracle.ring_allreduce_threads(xs, 5, S=S, bf16_acc=acc)
    for q in range(R):
        assert got[q].tobytes() == ref[q].tobytes(), f"threads, rank {q}"
    with pytest.raises(ValueError):
        oracle.ring_allreduce_range([x.copy() for x in xs], 0, n + 1, S, acc, part)


# a seeded sweep of the same invariants over random shapes (the GPU sweeps
# compare against the oracle over this whole space)
_SWEEP = [(int(R), int(n), int(S), dt, acc)
          for R, n, S, dt, acc in (
              (rng.choice([1, 2, 3, 4, 5, 7, 8, 13, 16, 31, 64]), int(10 ** rng.uniform(0, 4.3)),
               rng.integers(1, 9), *[("f32", "per_hop"), ("bf16", "per_hop"),
                                     ("bf16", "fp32_partials")][rng.integers(0, 3)])
              for rng in [np.random.default_rng(606)] for _ in range(150))]


@pytest.mark.parametrize("R,n,S,dt,acc", _SWEEP)
def test_invariants_random_shapes(R, n, S, dt, acc):
    xs = workloads.random_buffers(R, n, dt, seed=R * 31 + n, dist="normal", scale=1.0)
    ref = oracle.ring_allreduce(xs, S=S, bf16_acc=acc)
    one = oracle.ring_allreduce(xs, S=1, bf16_acc=acc)
    fold = oracle.fold(xs, bf16_acc=acc)
    for q in range(R):
        assert ref[q].tobytes() == fold.tobytes() and one[q].tobytes() == fold.tobytes()
    if n:
        idx = np.random.default_rng(n).integers(0, n, 64)
        np.testing.assert_array_equal(oracle.fold_at(xs, idx, bf16_acc=acc), fold[idx])
    vec = 4 if dt == "f32" else 8
    rs = oracle.ring_reduce_scatter(xs, S=S, bf16_acc=acc)
    for c in range(R):
        lo, hi = oracle.chunk_bounds(n, R, vec, c)
        np.testing.assert_array_equal(rs[c][lo:hi], fold[lo:hi])
    for q, b in enumerate(oracle.ring_all_gather(rs, S=S)):
        assert b.tobytes() == fold.tobytes(), f"rank {q}"
