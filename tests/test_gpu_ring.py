"""GPU parity of the ring all-reduce / reduce-scatter / all-gather against
the CPU oracle, element by element, bit for bit (fp32, and bf16 with per-hop
rounding: both sides apply the same deterministic rule)."""
import numpy as np
import pytest

import oracle
import workloads
from gpu_helpers import say, to_dev, to_host, torch_cuda

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ccr_mod():
    torch_cuda()
    import collective_communication_reduce_amd as ccr
    return ccr


@pytest.fixture(scope="module")
def ctx(ccr_mod):
    c = ccr_mod.Context(0, ccr_mod.Config())
    yield c
    c.close()


def _run(ccr, ctx, xs, which="allreduce"):
    import torch
    ts = [to_dev(x) for x in xs]
    getattr(ccr, f"ccr_{which}")(ctx, ts)
    torch.cuda.synchronize()
    return [to_host(t) for t in ts]


def _assert_bitwise(got, ref, what):
    for q, (g, r) in enumerate(zip(got, ref)):
        if g.tobytes() != r.tobytes():
            bad = np.nonzero(g != r)[0]
            raise AssertionError(f"{what}: rank {q} differs at {bad.size} elements, first {bad[:5]}")


CASES = [(1, 100), (2, 1), (2, 7), (3, 8), (3, 1000), (4, 4096 * 3 + 5), (5, 4099),
         (8, 65536 + 9), (17, 100003), (64, 2049), (7, 3)]


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("R,n", CASES)
@pytest.mark.parametrize("S", [1, 3])
def test_allreduce_bitwise(ccr_mod, ctx, dt, R, n, S):
    ctx.set_config(ccr_mod.Config(slices=S))
    xs = workloads.random_buffers(R, n, dt, seed=R * 131 + n, dist="normal", scale=1.0)
    say(f"allreduce {dt} R={R} n={n} S={S}")
    got = _run(ccr_mod, ctx, xs)
    _assert_bitwise(got, oracle.ring_allreduce(xs, S=S), f"allreduce {dt} R={R} n={n}")


SLICED = [(2, 17), (3, 1001), (7, 3), (5, 5 * 8192), (16, 4099), (33, 70001), (64, 131077),
          (2, 88)]  # bf16: whole-chunk slices 3-4 empty, the ragged chunk's slice 3 not


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("R,n", SLICED)
@pytest.mark.parametrize("S", [2, 5])
def test_sliced_ring_hops_bitwise(ccr_mod, ctx, dt, R, n, S):
    """Slices run as separate launches only when something overlaps them:
    with overlap on, every hop of slice s covers slice s of each chunk, so
    the ring-hop kernel's slice geometry is exercised (offsets inside whole
    chunks, the ragged chunk's own slices, empty slices of tiny chunks, the
    16-, 32- and 64-slot rank tables)."""
    ctx.set_config(ccr_mod.Config(overlap=True, slices=S))
    xs = workloads.random_buffers(R, n, dt, seed=R * 7 + n + S, dist="normal", scale=1.0)
    say(f"sliced allreduce {dt} R={R} n={n} S={S}")
    got = _run(ccr_mod, ctx, xs)
    _assert_bitwise(got, oracle.ring_allreduce(xs, S=S), f"sliced allreduce {dt} R={R} n={n} S={S}")
    rs = _run(ccr_mod, ctx, xs, "reduce_scatter")
    _assert_bitwise(rs, oracle.ring_reduce_scatter(xs, S=S), f"reduce_scatter {dt} R={R} n={n}")
    ctx.set_config(ccr_mod.Config())


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("R,n", [(3, 1000), (8, 65536 + 9), (32, 40961)])
def test_reduce_scatter_and_all_gather_bitwise(ccr_mod, ctx, dt, R, n):
    ctx.set_config(ccr_mod.Config(slices=2))
    xs = workloads.random_buffers(R, n, dt, seed=R + n, dist="uniform")
    say(f"reduce_scatter / all_gather {dt} R={R} n={n}")
    rs = _run(ccr_mod, ctx, xs, "reduce_scatter")
    _assert_bitwise(rs, oracle.ring_reduce_scatter(xs, S=2), "reduce_scatter")
    ag = _run(ccr_mod, ctx, xs, "all_gather")
    _assert_bitwise(ag, oracle.ring_all_gather(xs, S=2), "all_gather")


@pytest.mark.parametrize("R,n", [(2, 1000), (3, 8), (3, 1001), (5, 4099), (8, 65536 + 13), (17, 30011)])
@pytest.mark.parametrize("S", [1, 3])
@pytest.mark.parametrize("mode", [dict(), dict(overlap=True), dict(copy_mode="sdma")],
                         ids=["kernel", "overlap", "sdma"])
def test_bf16_fp32_partials_bitwise(ccr_mod, ctx, R, n, S, mode):
    """bf16 with the running partial carried in fp32 and rounded once."""
    ctx.set_config(ccr_mod.Config(slices=S, bf16_acc="fp32_partials", **mode))
    xs = workloads.random_buffers(R, n, "bf16", seed=R * 7 + n, dist="normal", scale=1.0)
    say(f"allreduce bf16 fp32-partials R={R} n={n} S={S} {mode}")
    got = _run(ccr_mod, ctx, xs)
    _assert_bitwise(got, oracle.ring_allreduce(xs, S=S, bf16_acc="fp32_partials"), "fp32 partials")
    rs = _run(ccr_mod, ctx, xs, "reduce_scatter")
    ref = oracle.ring_reduce_scatter(xs, S=S, bf16_acc="fp32_partials")
    for c in range(R):  # the owned chunks (the others hold per-hop scratch state)
        lo, hi = oracle.chunk_bounds(n, R, 8, c)
        np.testing.assert_array_equal(rs[c][lo:hi], ref[c][lo:hi])
    ctx.set_config(ccr_mod.Config())


MODES = [dict(overlap=True, slices=4), dict(copy_mode="sdma", slices=2),
         dict(copy_mode="sdma", overlap=True, slices=3), dict(cu_budget=64, slices=2),
         dict(cu_budget=16, overlap=True, slices=2, copy_mode="sdma"),
         dict(copy_mode="sdma", slices=2, dma_sync="stream_flags"),
         dict(copy_mode="sdma", slices=3, dma_engines=1), dict(copy_mode="sdma", dma_engines=4)]


@pytest.mark.parametrize("mode", MODES, ids=lambda m: "-".join(f"{k}={v}" for k, v in m.items()))
@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_modes_do_not_change_bits(ccr_mod, ctx, mode, dt):
    """Copy mode, overlap, slicing and CU budget leave the result bitwise
    unchanged."""
    ctx.set_config(ccr_mod.Config(**mode))
    R, n = 6, 3 * 65536 + 11
    xs = workloads.random_buffers(R, n, dt, seed=99, dist="normal", scale=1e-3)
    say(f"allreduce {dt} R={R} n={n} mode={mode}")
    got = _run(ccr_mod, ctx, xs)
    _assert_bitwise(got, oracle.ring_allreduce(xs, S=1), f"mode {mode}")
    rs = _run(ccr_mod, ctx, xs, "reduce_scatter")
    _assert_bitwise(rs, oracle.ring_reduce_scatter(xs, S=mode.get("slices", 1)), "reduce_scatter")
    ctx.set_config(ccr_mod.Config())


@pytest.mark.parametrize("place", ["static", "any"])
@pytest.mark.parametrize("R,n,engines", [(8, (1 << 20) + 24, 0), (5, 300007, 3), (16, 4096 * 64 + 8, 0)])
def test_sdma_engine_placement_does_not_change_bits(ccr_mod, ctx, monkeypatch, place, R, n, engines):
    """All-gather links on fixed engines or on the least-loaded engine when
    they become ready: the same bits as the oracle either way."""
    if place == "static":
        monkeypatch.setenv("CCR_DMA_PLACE", "static")
    else:
        monkeypatch.delenv("CCR_DMA_PLACE", raising=False)
    ctx.set_config(ccr_mod.Config(copy_mode="sdma", dma_engines=engines))
    xs = workloads.random_buffers(R, n, "bf16", seed=R + n, dist="normal", scale=1.0)
    say(f"allreduce sdma place={place} R={R} n={n} engines={engines}")
    got = _run(ccr_mod, ctx, xs)
    _assert_bitwise(got, oracle.ring_allreduce(xs, S=1), f"sdma placement {place}")
    ag_in = oracle.ring_reduce_scatter(xs, S=1)
    got = _run(ccr_mod, ctx, ag_in, "all_gather")
    _assert_bitwise(got, oracle.ring_all_gather(ag_in, S=1), f"sdma all-gather placement {place}")
    ctx.set_config(ccr_mod.Config())


def test_repeated_calls_on_one_stream(ccr_mod, ctx):
    """Back-to-back collectives on one stream see each other's results."""
    import torch
    ctx.set_config(ccr_mod.Config(slices=2, overlap=True))
    R, n = 4, 50000
    xs = workloads.integer_buffers(R, n, "f32", seed=5, bound=8)
    ts = [to_dev(x) for x in xs]
    say("two allreduces in a row")
    ccr_mod.ccr_allreduce(ctx, ts)
    ccr_mod.ccr_allreduce(ctx, ts)
    torch.cuda.synchronize()
    expect = R * np.sum(np.stack(xs), axis=0)
    for t in ts:
        np.testing.assert_array_equal(to_host(t), expect)
    ctx.set_config(ccr_mod.Config())


def test_invalid_arguments(ccr_mod, ctx):
    import torch
    a = torch.zeros(1000, device="cuda")
    b = torch.zeros(1000, device="cuda")
    say("invalid arguments")
    with pytest.raises(ccr_mod.CcrError) as e:   # misaligned (4-byte offset)
        ccr_mod.ccr_allreduce(ctx, [a[1:], b[1:]])
    assert "aligned" in str(e.value)
    with pytest.raises(ccr_mod.CcrError) as e:   # overlapping ranks
        ccr_mod.ccr_allreduce(ctx, [a[:500], a[400:900]])
    assert e.value.status == ccr_mod.CCR_ERR_INVALID_ARG
    host = np.zeros(1000, np.float32)
    import ctypes
    ptrs = (ctypes.c_void_p * 2)(host.ctypes.data, b.data_ptr())
    st = ccr_mod._lib.ccr_allreduce(ctx.handle, ptrs, 2, 1000, 0, None)
    assert st == ccr_mod.CCR_ERR_INVALID_ARG
    ptrs = (ctypes.c_void_p * 2)(a.data_ptr(), b.data_ptr())
    st = ccr_mod._lib.ccr_allreduce(ctx.handle, ptrs, 2, 1 << 34, 0, None)  # past the allocation
    assert st == ccr_mod.CCR_ERR_INVALID_ARG and "past the end" in ccr_mod.ccr_last_error()
    st = ccr_mod._lib.ccr_allreduce(ctx.handle, ptrs, 2, 1000, 5, None)
    assert st == ccr_mod.CCR_ERR_INVALID_ARG
    assert ccr_mod._lib.ccr_allreduce(ctx.handle, ptrs, 2, 0, 0, None) == ccr_mod.CCR_OK
    bad = ccr_mod.Config().to_c()
    bad.slices = 0
    import ctypes as ct
    assert ccr_mod._lib.ccr_ctx_set_config(ctx.handle, ct.byref(bad)) == ccr_mod.CCR_ERR_INVALID_ARG


@pytest.mark.parametrize("budget", [0, 32])
def test_profile_intervals(ccr_mod, budget):
    """Per-launch intervals follow the launches: ordered, inside the
    caller's window, and never holding more CUs than the budget allows."""
    import torch
    R, n = 8, 1 << 20
    xs = workloads.random_buffers(R, n, "f32", seed=9)
    ts = [to_dev(x) for x in xs]
    say(f"profile intervals, cu_budget={budget}")
    with ccr_mod.Context(0, ccr_mod.Config(cu_budget=budget)) as c:
        ccr_mod.ccr_allreduce(c, ts)
        torch.cuda.synchronize()
        ccr_mod.ccr_profile_enable(c, True)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        ccr_mod.ccr_allreduce(c, ts)
        e1.record()
        torch.cuda.synchronize()
        window = e0.elapsed_time(e1)
        red = ccr_mod.ccr_profile_intervals(c, "reduce", e0)
        fwd = ccr_mod.ccr_profile_intervals(c, "reduce_forward", e0)
        cpy = ccr_mod.ccr_profile_intervals(c, "copy_kernel", e0)
        stats = ccr_mod.ccr_profile_read(c, "reduce")
        ccr_mod.ccr_profile_enable(c, False)
    assert (len(red), len(fwd), len(cpy)) == (R - 2, 1, R - 2) == (stats["launches"], 1, R - 2)
    allowed = budget or torch.cuda.get_device_properties(0).multi_processor_count
    iv = np.concatenate([red, fwd, cpy])
    assert (iv[:, 0] >= -1e-3).all() and (iv[:, 1] >= iv[:, 0]).all() and (iv[:, 1] <= window + 1e-3).all()
    assert (iv[:, 2] >= 1).all() and (iv[:, 2] <= allowed).all()
    assert (iv[:, 2] == allowed).all()  # 1 Mi elements per rank: far more workgroups than CUs
    hops = np.concatenate([red, fwd, cpy])
    hops = hops[np.argsort(hops[:, 0])]
    assert (np.diff(hops[:, 0]) > 0).all()  # one stream: launches run one after another
    assert abs(np.sum(red[:, 1] - red[:, 0]) - stats["ms"]) < 1e-2


@pytest.mark.parametrize("env", [{"HIP_LAUNCH_BLOCKING": "1"}, {"CCR_NONTEMPORAL": "0"},
                                 {"CCR_NONTEMPORAL": "1"}, {"CCR_NONTEMPORAL": "2"},
                                 {"CCR_RING_HOPS": "table"}, {"CCR_GRID": "64"}],
                         ids=lambda e: "-".join(f"{k}={v}" for k, v in e.items()))
def test_process_settings_do_not_change_bits(ccr_mod, tmp_path, env):
    """Settings read once per process leave the bits unchanged in every
    mode: HIP_LAUNCH_BLOCKING=1 (every launch waits for the previous one),
    each forced non-temporal mode of the streaming kernels (none, every
    load and store, the incoming load only), ring hops launched from the
    piece table instead of the rank base addresses, and piece-table launches
    capped at 64 workgroups, each looping over many tiles (the form every
    launch past one dispatch's 2^24 - 1 workgroups takes).  Each case runs
    in a child process of its own."""
    import os
    import subprocess
    import sys
    R, n = 5, 2 * 65536 + 7
    xs = workloads.random_buffers(R, n, "bf16", seed=77, dist="normal", scale=1e-3)
    src, dst = tmp_path / "in.npz", tmp_path / "out.npz"
    np.savez(src, R=R, **{f"x{i}": x for i, x in enumerate(xs)})
    say(f"child process {env} R={R} n={n}")
    child = os.path.join(os.path.dirname(__file__), "launch_blocking_child.py")
    r = subprocess.run([sys.executable, child, str(src), str(dst)], env=dict(os.environ, **env),
                       timeout=150, capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    got = np.load(dst)
    ref = oracle.ring_allreduce(xs, S=1)
    for name in ("kernel_s1", "kernel_overlap_s3", "sdma_s2"):
        _assert_bitwise([got[f"{name}_{q}"] for q in range(R)], ref, f"{env}, {name}")
    _assert_bitwise([got[f"sendrecv_{q}"] for q in range(R)], [x[: n // 8 * 8] for x in xs],
                    f"{env}, sendrecv")


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_past_32_bit_offsets(ccr_mod, dt):
    """3 ranks of 2^31 + 12345 elements (4 or 8 GiB each): element indices
    past 2^31 and byte offsets past 4 GiB.  Inputs come from torch's seeded
    generator on the device; sampled outputs (chunk edges, the 2^31
    boundary, the ragged end, random picks) must equal the oracle's fold of
    the same input values bit for bit, on every rank.  An element of chunk c
    folds ranks c+1, ..., c-1 and then c, so the oracle folds each sample's
    values rotated by c."""
    import torch
    R, n = 3, (1 << 31) + 12345
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    vec = 8 if dt == "bf16" else 4
    say(f"allreduce {dt} R={R} n={n} (past 32-bit offsets)")
    gen = torch.Generator(device="cuda").manual_seed(31)
    bufs = []
    for _ in range(R):
        x = torch.empty(n, dtype=tdt, device="cuda")
        for lo in range(0, n, 1 << 28):  # draw in float32 pieces, cast in place
            hi = min(n, lo + (1 << 28))
            x[lo:hi] = torch.randn(hi - lo, generator=gen, device="cuda").mul_(1e-3).to(tdt)
        bufs.append(x)
    rng = np.random.default_rng(5)
    edges = [0, 1, n - 1, n - 2, (1 << 31) - 1, 1 << 31, (1 << 31) + 1]
    for c in range(R):
        lo, hi = oracle.chunk_bounds(n, R, vec, c)
        edges += [lo, max(lo, hi - 1)]
    idx = np.unique(np.concatenate([np.array(edges, np.int64), rng.integers(0, n, 2000)]))
    d_idx = torch.from_numpy(idx).cuda()
    before = [to_host(b[d_idx]) for b in bufs]
    with ccr_mod.Context(0) as c:
        ccr_mod.ccr_allreduce(c, bufs)
        torch.cuda.synchronize()
    after = [to_host(b[d_idx]) for b in bufs]
    del bufs
    torch.cuda.empty_cache()
    chunk = np.zeros(idx.size, np.int64)
    for c in range(R):
        lo, hi = oracle.chunk_bounds(n, R, vec, c)
        chunk[(idx >= lo) & (idx < hi)] = c
    want = np.empty_like(before[0])
    for k in range(idx.size):
        cc = int(chunk[k])
        rot = [before[(r + cc) % R][k:k + 1] for r in range(R)]
        want[k] = oracle.fold(rot)[0]
    for q in range(R):
        assert after[q].tobytes() == want.tobytes(), f"rank {q} differs from the oracle"


# ------------------------------------------------ full-size workloads
FULL = [(workloads.RING_SMALL_F32, "allreduce"), (workloads.DP_BUCKET_BF16, "allreduce"),
        (workloads.RS_AG_R32_F32, "rs_then_ag")]


@pytest.mark.parametrize("w,how", FULL, ids=[w.name for w, _ in FULL])
def test_full_size_workloads(ccr_mod, w, how):
    """The benchmark's sizes and launch configuration, compared bit for bit
    with the oracle's closed-form fold on every element (the bf16 bucket also
    with fp32 partials)."""
    import torch
    say(f"full-size {w.name}: generating inputs")
    xs = workloads.ring_inputs(w)
    ref = oracle.fold(xs)
    say(f"full-size {w.name}: running on the GPU (S={w.slices})")
    with ccr_mod.Context(0, ccr_mod.Config(slices=w.slices)) as c:
        ts = [to_dev(x) for x in xs]
        if how == "allreduce":
            ccr_mod.ccr_allreduce(c, ts)
        else:
            ccr_mod.ccr_reduce_scatter(c, ts)
            ccr_mod.ccr_all_gather(c, ts)
        torch.cuda.synchronize()
        for q, t in enumerate(ts):
            g = to_host(t)
            if g.tobytes() != ref.tobytes():
                bad = np.nonzero(g != ref)[0]
                raise AssertionError(f"{w.name}: rank {q} differs at {bad.size} elements")
    if w.dtype == "bf16":
        exact = np.zeros(w.count, np.float64)
        for x in xs:
            exact += oracle.bf16_to_f32(x)
        err = np.max(np.abs(oracle.bf16_to_f32(ref) - exact)) / np.max(np.abs(exact))
        say(f"{w.name}: normalised max error vs fp64 = {err:.4f}")
        assert err <= 1e-2
        ref32 = oracle.fold(xs, bf16_acc="fp32_partials")
        with ccr_mod.Context(0, ccr_mod.Config(slices=w.slices, bf16_acc="fp32_partials")) as c:
            ts = [to_dev(x) for x in xs]
            ccr_mod.ccr_allreduce(c, ts)
            torch.cuda.synchronize()
            for q, t in enumerate(ts):
                assert to_host(t).tobytes() == ref32.tobytes(), f"fp32 partials, rank {q}"
        err32 = np.max(np.abs(oracle.bf16_to_f32(ref32) - exact)) / np.max(np.abs(exact))
        say(f"{w.name}: fp32 partials normalised max error vs fp64 = {err32:.4f}")
        assert err32 <= err


# SDMA all-gathers at the gradient bucket's full size, in the settings the
# benchmark times under its GEMM load: every engine with least-loaded link
# placement, engine caps (8 and 2), and deadline pacing.
SDMA_FULL = [dict(copy_mode="sdma"), dict(copy_mode="sdma", dma_engines=8),
             dict(copy_mode="sdma", dma_engines=2), dict(copy_mode="sdma", dma_deadline_us=3000)]


@pytest.fixture(scope="module")
def bucket_inputs():
    w = workloads.DP_BUCKET_BF16
    say(f"full-size {w.name}: generating inputs and the oracle's fold")
    xs = workloads.ring_inputs(w)
    return xs, oracle.fold(xs)


@pytest.mark.parametrize("cfg", SDMA_FULL, ids=lambda c: "-".join(f"{k}={v}" for k, v in c.items()))
def test_full_size_bucket_with_sdma_all_gather(ccr_mod, bucket_inputs, cfg):
    """8 ranks x 25 Mi bf16: every element of every rank equals the oracle's
    fold, with the all-gather on the SDMA engines (links of up to 8 MiB cut
    into sub-chains and placed on the least-loaded engine as they become
    ready)."""
    import torch
    xs, ref = bucket_inputs
    w = workloads.DP_BUCKET_BF16
    say(f"full-size {w.name} with {cfg}")
    with ccr_mod.Context(0, ccr_mod.Config(slices=w.slices, **cfg)) as c:
        ts = [to_dev(x) for x in xs]
        ccr_mod.ccr_allreduce(c, ts)
        torch.cuda.synchronize()
        used = ccr_mod.ccr_dma_rate(c)[1]
        for q, t in enumerate(ts):
            g = to_host(t)
            if g.tobytes() != ref.tobytes():
                bad = np.nonzero(g != ref)[0]
                raise AssertionError(f"{cfg}: rank {q} differs at {bad.size} elements, first {bad[:5]}")
    if "dma_engines" in cfg:
        assert used <= cfg["dma_engines"]


def test_full_size_rs_then_sdma_all_gather_r32(ccr_mod):
    """32 ranks x 8 Mi fp32 (1 GiB): the reduce-scatter call, then the
    all-gather call with SDMA copies; every element equals the oracle's fold."""
    import torch
    w = workloads.RS_AG_R32_F32
    say(f"full-size {w.name}: generating inputs")
    xs = workloads.ring_inputs(w)
    ref = oracle.fold(xs)
    say(f"full-size {w.name}: reduce-scatter, then SDMA all-gather (S={w.slices})")
    with ccr_mod.Context(0, ccr_mod.Config(slices=w.slices, copy_mode="sdma")) as c:
        ts = [to_dev(x) for x in xs]
        del xs
        ccr_mod.ccr_reduce_scatter(c, ts)
        ccr_mod.ccr_all_gather(c, ts)
        torch.cuda.synchronize()
        for q, t in enumerate(ts):
            g = to_host(t)
            if g.tobytes() != ref.tobytes():
                bad = np.nonzero(g != ref)[0]
                raise AssertionError(f"rank {q} differs at {bad.size} elements, first {bad[:5]}")
