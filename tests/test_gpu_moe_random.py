"""Seeded random sweep of the MoE calls, each case checked against the oracle
as the fixed-size MoE tests check theirs (routing, plan, every buffer of the
three-stage dispatch byte for byte, the combine returning every token to all
K of its slots; the fused gather's expert-major rows byte for byte): 1-16
ranks, 1-16 experts per rank, top-1 to top-16, 1 to ~1,500 tokens, rows of
16 B to 1 KiB, kernel or SDMA exchange, and fused calls with skewed routing
(destinations left without rows) or repeated on the same plan.  The cases
are fixed by the seed."""
import numpy as np
import pytest

from gpu_helpers import torch_cuda
from test_gpu_moe import _dispatch_case, _fused_case

pytestmark = pytest.mark.gpu

N_CASES = 200


def _cases(seed=4242):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(N_CASES):
        R = int(rng.choice([1, 2, 3, 4, 5, 8, 16]))
        E = R * int(rng.integers(1, 17))
        if E > 1024:
            E = R * (1024 // R)
        K = int(rng.integers(1, min(E, 16) + 1))
        T = int(10 ** rng.uniform(0, 3.2))
        H = 8 * int(rng.integers(1, 65))
        kind = str(rng.choice(["kernel", "sdma", "fused", "fused"]))
        skew = int(rng.integers(1, R + 1)) if kind == "fused" and rng.random() < 0.3 else None
        reps = 2 if kind == "fused" and rng.random() < 0.2 else 1
        out.append((i, R, T, E, K, H, kind, skew, reps))
    return out


CASES = _cases()


@pytest.fixture(scope="module")
def ccr_mod():
    torch_cuda()
    import collective_communication_reduce_amd as ccr
    return ccr


@pytest.mark.parametrize("case", CASES, ids=[f"case{c[0]}-{c[6]}" for c in CASES])
def test_random_moe_case(ccr_mod, case):
    i, R, T, E, K, H, kind, skew, reps = case
    if kind == "fused":
        _fused_case(ccr_mod, R, T, E, K, H, skew=skew, reps=reps)
    else:
        _dispatch_case(ccr_mod, R, T, E, K, H, kind)
