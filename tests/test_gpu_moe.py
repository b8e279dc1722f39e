"""GPU parity of expert-parallel MoE dispatch/combine against the CPU
oracle: routing and plan indices bit-exact, every buffer byte-exact, and the
round trip returns every token to every one of its K slots."""
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


@pytest.mark.parametrize("T,E,K", [(1, 8, 1), (64, 16, 4), (4096, 64, 6), (100, 1024, 16), (33, 200, 7)])
def test_topk_bitwise(ccr_mod, T, E, K):
    import torch
    rng = np.random.default_rng(T + E)
    logits = (np.round(rng.normal(0, 1, (T, E)) * 4) / 4).astype(np.float32)  # many ties
    say(f"moe_topk T={T} E={E} K={K}")
    with ccr_mod.Context(0) as c:
        out = torch.zeros(T, K, dtype=torch.int32, device="cuda")
        ccr_mod.ccr_moe_topk(c, torch.from_numpy(logits).cuda(), out)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(to_host(out), oracle.moe_topk(logits, K))


def _dispatch_case(ccr_mod, R, T, E, K, H, mode, seed=0):
    import torch
    w = workloads.MOE_DISPATCH_BF16
    xs, logits = workloads.moe_inputs(w, tokens=T, R=R)
    xs = [x[:, :H].copy() for x in xs]
    logits = [l[:, :E].copy() if E <= l.shape[1] else np.tile(l, (1, -(-E // l.shape[1])))[:, :E].copy()
              for l in logits]
    ref_topk = [oracle.moe_topk(l, K) for l in logits]
    ref = oracle.moe_dispatch(xs, ref_topk, E)
    say(f"moe dispatch/combine R={R} T={T} E={E} K={K} H={H} mode={mode}")
    with ccr_mod.Context(0, ccr_mod.Config(copy_mode=mode)) as c:
        d_x = [to_dev(x) for x in xs]
        topk = [torch.zeros(T, K, dtype=torch.int32, device="cuda") for _ in range(R)]
        src_tok = [torch.zeros(T * K, dtype=torch.int32, device="cuda") for _ in range(R)]
        slot = [torch.zeros(T * K, dtype=torch.int32, device="cuda") for _ in range(R)]
        ecnt = []
        for r in range(R):
            ccr_mod.ccr_moe_topk(c, to_dev(logits[r]), topk[r])
            ecnt.append(ccr_mod.ccr_moe_plan(c, topk[r], E, R, src_tok[r], slot[r]))
        ecnt = np.stack(ecnt)
        for r in range(R):
            np.testing.assert_array_equal(to_host(topk[r]), ref_topk[r])
            np.testing.assert_array_equal(to_host(src_tok[r]), ref["src_tok"][r])
            np.testing.assert_array_equal(to_host(slot[r]).reshape(T, K), ref["slot"][r])
        np.testing.assert_array_equal(ecnt, ref["ecnt"])
        rows = [int(ref["counts"][:, d].sum()) for d in range(R)]
        send = [torch.zeros(T * K, H, dtype=torch.bfloat16, device="cuda") for _ in range(R)]
        recv = [torch.zeros(max(1, n), H, dtype=torch.bfloat16, device="cuda") for n in rows]
        exp = [torch.zeros(max(1, n), H, dtype=torch.bfloat16, device="cuda") for n in rows]
        ccr_mod.ccr_moe_dispatch(c, d_x, src_tok, ecnt, K, send, recv, exp)
        torch.cuda.synchronize()
        for r in range(R):
            np.testing.assert_array_equal(to_host(send[r]), ref["send"][r])
        for d in range(R):
            np.testing.assert_array_equal(to_host(recv[d])[:rows[d]], ref["recv"][d])
            np.testing.assert_array_equal(to_host(exp[d])[:rows[d]], ref["exp"][d])
        out = [torch.zeros(T, K, H, dtype=torch.bfloat16, device="cuda") for _ in range(R)]
        recv2 = [torch.zeros_like(x) for x in recv]
        send2 = [torch.zeros_like(x) for x in send]
        ccr_mod.ccr_moe_combine(c, exp, slot, ecnt, T, K, recv2, send2, out)
        torch.cuda.synchronize()
        for r in range(R):
            o = to_host(out[r])
            np.testing.assert_array_equal(o, np.repeat(xs[r][:, None, :], K, axis=1))


@pytest.mark.parametrize("mode", ["kernel", "sdma"])
@pytest.mark.parametrize("R,T,E,K,H", [(2, 4, 4, 2, 8), (2, 50, 8, 2, 64), (4, 257, 16, 3, 136),
                                       (8, 512, 64, 6, 256)])
def test_dispatch_combine_small(ccr_mod, mode, R, T, E, K, H):
    _dispatch_case(ccr_mod, R, T, E, K, H, mode)


@pytest.mark.parametrize("mode", ["kernel", "sdma"])
def test_dispatch_combine_full_size(ccr_mod, mode):
    """8 ranks x 4096 tokens x 2048 hidden bf16, 64 experts, top-6."""
    w = workloads.MOE_DISPATCH_BF16
    _dispatch_case(ccr_mod, w.R, w.tokens, w.experts, w.topk, w.hidden, mode)


def _plan(ccr_mod, c, logits, E, K, R):
    import torch
    T = logits[0].shape[0]
    topk = [torch.zeros(T, K, dtype=torch.int32, device="cuda") for _ in range(R)]
    src_tok = [torch.zeros(T * K, dtype=torch.int32, device="cuda") for _ in range(R)]
    slot = [torch.zeros(T * K, dtype=torch.int32, device="cuda") for _ in range(R)]
    ecnt = []
    for r in range(R):
        ccr_mod.ccr_moe_topk(c, to_dev(logits[r]), topk[r])
        ecnt.append(ccr_mod.ccr_moe_plan(c, topk[r], E, R, src_tok[r], slot[r]))
    return src_tok, slot, np.stack(ecnt)


def _fused_case(ccr_mod, R, T, E, K, H, skew=None, reps=1):
    """Fused dispatch: exp byte-exact against the oracle's three-stage
    dispatch; fused combine: every token back in all K of its slots."""
    import torch
    w = workloads.MOE_DISPATCH_BF16
    xs, logits = workloads.moe_inputs(w, tokens=T, R=R)
    xs = [x[:, :H].copy() for x in xs]
    logits = [np.tile(l, (1, -(-E // l.shape[1])))[:, :E].copy() for l in logits]
    if skew is not None:  # route every token of the first ranks to the lowest experts
        for r in range(min(skew, R)):
            logits[r][:, :K] += 100.0
    ref_topk = [oracle.moe_topk(l, K) for l in logits]
    ref = oracle.moe_dispatch(xs, ref_topk, E)
    say(f"moe fused dispatch/combine R={R} T={T} E={E} K={K} H={H} skew={skew} reps={reps}")
    with ccr_mod.Context(0) as c:
        src_tok, slot, ecnt = _plan(ccr_mod, c, logits, E, K, R)
        np.testing.assert_array_equal(ecnt, ref["ecnt"])
        rows = [int(ref["counts"][:, d].sum()) for d in range(R)]
        d_x = [to_dev(x) for x in xs]
        for rep in range(reps):
            # a destination with no rows gets an empty tensor (its pointer may be NULL)
            exp = [torch.full((n, H), -7.0, dtype=torch.bfloat16, device="cuda") for n in rows]
            ccr_mod.ccr_moe_dispatch_fused(c, d_x, src_tok, ecnt, K, exp)
            out = [torch.zeros(T, K, H, dtype=torch.bfloat16, device="cuda") for _ in range(R)]
            ccr_mod.ccr_moe_combine_fused(c, exp, slot, ecnt, T, K, out)
            torch.cuda.synchronize()
            for d in range(R):
                np.testing.assert_array_equal(to_host(exp[d]), ref["exp"][d].reshape(rows[d], H))
            for r in range(R):
                np.testing.assert_array_equal(to_host(out[r]), np.repeat(xs[r][:, None, :], K, axis=1))


@pytest.mark.parametrize("R,T,E,K,H", [(1, 5, 4, 2, 8), (2, 4, 4, 2, 8), (2, 50, 8, 2, 64),
                                       (4, 257, 16, 3, 136), (8, 512, 64, 6, 256),
                                       (3, 1, 6, 6, 8), (5, 77, 1000, 16, 24)])
def test_fused_dispatch_combine_small(ccr_mod, R, T, E, K, H):
    _fused_case(ccr_mod, R, T, E, K, H)


def test_fused_dispatch_empty_destinations(ccr_mod):
    # ranks 0..3 send every row to experts 0..K-1, which live on rank 0
    _fused_case(ccr_mod, 4, 100, 8, 2, 64, skew=4)


def test_fused_repeated_calls_reuse_tables(ccr_mod):
    # more calls than table slots, each checked
    _fused_case(ccr_mod, 4, 129, 16, 4, 72, reps=6)
    _fused_case(ccr_mod, 2, 31, 4, 1, 16, reps=2)


def test_fused_dispatch_combine_full_size(ccr_mod):
    """8 ranks x 4096 tokens x 2048 hidden bf16, 64 experts, top-6."""
    w = workloads.MOE_DISPATCH_BF16
    _fused_case(ccr_mod, w.R, w.tokens, w.experts, w.topk, w.hidden)


def test_fused_invalid_arguments(ccr_mod):
    import torch
    R, T, E, K, H = 2, 16, 4, 2, 8
    w = workloads.MOE_DISPATCH_BF16
    xs, logits = workloads.moe_inputs(w, tokens=T, R=R)
    xs = [x[:, :H].copy() for x in xs]
    logits = [l[:, :E].copy() for l in logits]
    say("moe fused invalid arguments")
    with ccr_mod.Context(0) as c:
        src_tok, slot, ecnt = _plan(ccr_mod, c, logits, E, K, R)
        rows = [int(ecnt[:, (E // R) * d:(E // R) * (d + 1)].sum()) for d in range(R)]
        d_x = [to_dev(x) for x in xs]
        exp = [torch.zeros(max(1, n), H, dtype=torch.bfloat16, device="cuda") for n in rows]
        # an expert-major buffer that overlaps a source
        big = torch.zeros(T + max(rows) + 1, H, dtype=torch.bfloat16, device="cuda")
        with pytest.raises(ccr_mod.CcrError) as e:
            ccr_mod.ccr_moe_dispatch_fused(c, [big[:T], d_x[1]], src_tok, ecnt, K, [big[1:], exp[1]])
        assert e.value.status == ccr_mod.CCR_ERR_INVALID_ARG
        # counts that do not add up to T*K
        bad = ecnt.copy()
        bad[0, 0] += 1
        with pytest.raises(ccr_mod.CcrError):
            ccr_mod.ccr_moe_dispatch_fused(c, d_x, src_tok, bad, K, exp)
        # two outputs of the combine that overlap
        out = torch.zeros(2 * T * K + 1, H, dtype=torch.bfloat16, device="cuda")
        with pytest.raises(ccr_mod.CcrError):
            ccr_mod.ccr_moe_combine_fused(c, exp, slot, ecnt, T, K, [out[:T * K], out[1:T * K + 1]])
        # the valid call still works afterwards
        ccr_mod.ccr_moe_dispatch_fused(c, d_x, src_tok, ecnt, K, exp)
        torch.cuda.synchronize()


def test_overlapping_buffers_rejected(ccr_mod):
    """A buffer a call writes may not overlap another buffer of the call,
    index arrays included; the three-stage and the fused paths alike."""
    import torch
    R, T, E, K, H = 2, 16, 4, 2, 8
    w = workloads.MOE_DISPATCH_BF16
    xs, logits = workloads.moe_inputs(w, tokens=T, R=R)
    xs = [x[:, :H].copy() for x in xs]
    logits = [l[:, :E].copy() for l in logits]
    say("moe overlapping buffers")
    with ccr_mod.Context(0) as c:
        src_tok, slot, ecnt = _plan(ccr_mod, c, logits, E, K, R)
        rows = [int(ecnt[:, (E // R) * d:(E // R) * (d + 1)].sum()) for d in range(R)]
        d_x = [to_dev(x) for x in xs]
        send = [torch.zeros(T * K, H, dtype=torch.bfloat16, device="cuda") for _ in range(R)]
        recv = [torch.zeros(max(1, n), H, dtype=torch.bfloat16, device="cuda") for n in rows]
        exp = [torch.zeros(max(1, n), H, dtype=torch.bfloat16, device="cuda") for n in rows]

        def rejected(fn, *a):
            with pytest.raises(ccr_mod.CcrError) as e:
                fn(c, *a)
            assert e.value.status == ccr_mod.CCR_ERR_INVALID_ARG
            assert "overlap" in ccr_mod.ccr_last_error()

        # dispatch: send over x, recv over send, exp over recv
        big = torch.zeros(T * K + T, H, dtype=torch.bfloat16, device="cuda")
        rejected(ccr_mod.ccr_moe_dispatch, [big[:T], d_x[1]], src_tok, ecnt, K,
                 [big[T - 1:T - 1 + T * K], send[1]], recv, exp)
        both = torch.zeros(T * K + max(rows), H, dtype=torch.bfloat16, device="cuda")
        rejected(ccr_mod.ccr_moe_dispatch, d_x, src_tok, ecnt, K,
                 [both[:T * K], send[1]], [both[T * K - 1:T * K - 1 + rows[0]], recv[1]], exp)
        # an expert-major output that runs into the index array
        combo = torch.zeros(T * K + rows[0] * H // 2, dtype=torch.int32, device="cuda")
        combo[:T * K] = src_tok[0]
        exp0 = combo[T * K - 4:T * K - 4 + rows[0] * H // 2].view(torch.bfloat16).view(rows[0], H)
        rejected(ccr_mod.ccr_moe_dispatch_fused, d_x, [combo[:T * K], src_tok[1]], ecnt, K,
                 [exp0, exp[1]])
        # combine: out over send
        outs = torch.zeros(T * K + T * K, H, dtype=torch.bfloat16, device="cuda")
        rejected(ccr_mod.ccr_moe_combine, exp, slot, ecnt, T, K, recv,
                 [outs[:T * K], send[1]],
                 [outs[T * K - 1:2 * T * K - 1].view(T, K, H), torch.zeros(T, K, H, dtype=torch.bfloat16, device="cuda")])
        # the valid calls still work and give the three-stage placement
        ccr_mod.ccr_moe_dispatch(c, d_x, src_tok, ecnt, K, send, recv, exp)
        exp2 = [torch.zeros_like(e) for e in exp]
        ccr_mod.ccr_moe_dispatch_fused(c, d_x, src_tok, ecnt, K, exp2)
        torch.cuda.synchronize()
        for d in range(R):
            assert torch.equal(exp[d][:rows[d]], exp2[d][:rows[d]])
