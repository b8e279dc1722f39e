"""Out-of-bounds guards: every operand sits between two 4 KiB guard regions
filled with a known byte pattern; after the call the guards must be intact.
Ragged sizes exercise the kernels' tail handling."""
import numpy as np
import pytest

import workloads
from gpu_helpers import say, to_dev, torch_cuda

pytestmark = pytest.mark.gpu

GUARD = 4096  # bytes on each side; keeps the operand 16-byte aligned


@pytest.fixture(scope="module")
def ccr_mod():
    torch_cuda()
    import collective_communication_reduce_amd as ccr
    return ccr


def guarded(nbytes, fill=None):
    """(whole uint8 tensor, operand view) with the operand in the middle."""
    import torch
    whole = torch.full((GUARD + nbytes + GUARD,), 0xA5, dtype=torch.uint8, device="cuda")
    body = whole[GUARD:GUARD + nbytes]
    if fill is not None:
        body.copy_(fill)
    return whole, body


def intact(whole, nbytes):
    import torch
    g = torch.cat([whole[:GUARD], whole[GUARD + nbytes:]])
    return bool((g == 0xA5).all())


@pytest.mark.parametrize("which", ["allreduce", "reduce_scatter", "all_gather"])
@pytest.mark.parametrize("dt,R,n", [("f32", 3, 1001), ("bf16", 5, 4099), ("bf16", 8, 65536 + 13),
                                    ("f32", 7, 3), ("bf16", 2, 1)])
@pytest.mark.parametrize("mode", [dict(), dict(copy_mode="sdma", slices=2),
                                  dict(bf16_acc="fp32_partials", overlap=True, slices=3)],
                         ids=["kernel", "sdma", "partials-overlap"])
def test_ring_guards(ccr_mod, which, dt, R, n, mode):
    import torch
    xs = workloads.random_buffers(R, n, dt, seed=R * 7 + n)
    esize = 2 if dt == "bf16" else 4
    say(f"guards {which} {dt} R={R} n={n} {mode}")
    wholes, views = [], []
    for x in xs:
        w, b = guarded(n * esize, to_dev(x).view(torch.uint8))
        wholes.append(w)
        views.append(b.view(torch.bfloat16 if dt == "bf16" else torch.float32))
    with ccr_mod.Context(0, ccr_mod.Config(**mode)) as c:
        getattr(ccr_mod, f"ccr_{which}")(c, views)
        torch.cuda.synchronize()
    for q, w in enumerate(wholes):
        assert intact(w, n * esize), f"rank {q}: a guard byte changed"


@pytest.mark.parametrize("mode", ["kernel", "sdma"])
def test_staging_and_alltoall_guards(ccr_mod, mode):
    import torch
    say(f"guards sendrecv / alltoall {mode}")
    rng = np.random.default_rng(3)
    with ccr_mod.Context(0, ccr_mod.Config(copy_mode=mode, staging_chunk_bytes=4096,
                                           staging_slots=2)) as c:
        nbytes = 4096 * 3 + 48
        src = [guarded(nbytes, torch.from_numpy(rng.integers(0, 256, nbytes, dtype=np.uint8)).cuda())
               for _ in range(3)]
        dst = [guarded(nbytes) for _ in range(3)]
        ccr_mod.ccr_sendrecv_batch(c, [b for _, b in src], [b for _, b in dst])
        torch.cuda.synchronize()
        for (w, b), (_, s) in zip(dst, src):
            assert intact(w, nbytes) and torch.equal(b, s)
        R, row = 4, 48
        counts = rng.integers(0, 6, (R, R))
        sizes = [int(counts[r].sum()) * row for r in range(R)]
        rsizes = [int(counts[:, d].sum()) * row for d in range(R)]
        send = [guarded(sz, torch.from_numpy(rng.integers(0, 256, sz, dtype=np.uint8)).cuda()) for sz in sizes]
        recv = [guarded(sz) for sz in rsizes]
        ccr_mod.ccr_alltoall_rows(c, [b for _, b in send], [b for _, b in recv], counts, row)
        torch.cuda.synchronize()
        for (w, _), sz in zip(recv + send, rsizes + sizes):
            assert intact(w, sz)


def test_fused_moe_guards(ccr_mod):
    import torch
    R, T, E, K, H = 4, 77, 8, 3, 24  # 48-byte rows: 3 vectors, fewer than one per thread
    w = workloads.MOE_DISPATCH_BF16
    xs, logits = workloads.moe_inputs(w, tokens=T, R=R)
    say("guards fused MoE dispatch / combine")
    row = H * 2
    with ccr_mod.Context(0) as c:
        topk = [torch.zeros(T, K, dtype=torch.int32, device="cuda") for _ in range(R)]
        src_tok = [torch.zeros(T * K, dtype=torch.int32, device="cuda") for _ in range(R)]
        slot = [torch.zeros(T * K, dtype=torch.int32, device="cuda") for _ in range(R)]
        ecnt = []
        for r in range(R):
            ccr_mod.ccr_moe_topk(c, to_dev(logits[r][:, :E].copy()), topk[r])
            ecnt.append(ccr_mod.ccr_moe_plan(c, topk[r], E, R, src_tok[r], slot[r]))
        ecnt = np.stack(ecnt)
        rows = [int(ecnt[:, (E // R) * d:(E // R) * (d + 1)].sum()) for d in range(R)]
        x = [guarded(T * row, to_dev(xs[r][:, :H].copy()).view(torch.uint8).reshape(-1)) for r in range(R)]
        exp = [guarded(n * row) for n in rows]
        out = [guarded(T * K * row) for _ in range(R)]
        xv = [b.view(torch.bfloat16).reshape(T, H) for _, b in x]
        ev = [b.view(torch.bfloat16).reshape(n, H) for (_, b), n in zip(exp, rows)]
        ov = [b.view(torch.bfloat16).reshape(T, K, H) for _, b in out]
        ccr_mod.ccr_moe_dispatch_fused(c, xv, src_tok, ecnt, K, ev)
        ccr_mod.ccr_moe_combine_fused(c, ev, slot, ecnt, T, K, ov)
        torch.cuda.synchronize()
        for (wt, _), sz in zip(x + exp + out, [T * row] * R + [n * row for n in rows] + [T * K * row] * R):
            assert intact(wt, sz)
        for r in range(R):
            assert torch.equal(ov[r], xv[r][:, None, :].expand(T, K, H))
