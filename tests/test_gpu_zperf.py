"""The reduce path's bandwidth target, checked on the full gradient bucket
(8 ranks x 25 Mi bf16): the plain reduce-scatter hop reaches at least 70%
of the MI355X's 8 TB/s HBM peak, counting the hop's algorithmic bytes (read
local, read incoming, write local) over the kernel's own duration, taken
from events attached to each launch.  Collected last among the GPU tests."""
import pytest

import workloads
from gpu_helpers import say, to_dev, torch_cuda

pytestmark = pytest.mark.gpu

HBM_PEAK_GBS = 8000.0


def test_reduce_hop_reaches_70_percent_of_hbm_peak():
    torch_cuda()
    import torch
    import collective_communication_reduce_amd as ccr
    w = workloads.DP_BUCKET_BF16
    bufs = [to_dev(x) for x in workloads.ring_inputs(w)]
    with ccr.Context(0) as c:
        for _ in range(3):
            ccr.ccr_allreduce(c, bufs)
        ccr.ccr_profile_enable(c, True)
        for _ in range(10):
            ccr.ccr_allreduce(c, bufs)
        red = ccr.ccr_profile_read(c, "reduce")
        ccr.ccr_profile_enable(c, False)
        torch.cuda.synchronize()
    gbs = red["bytes"] / (red["ms"] * 1e6)
    say(f"reduce hop: {red['launches']} launches, {gbs:.0f} GB/s = {gbs / HBM_PEAK_GBS:.1%} of 8 TB/s")
    assert red["launches"] == 10 * (w.R - 2)
    assert gbs >= 0.70 * HBM_PEAK_GBS
