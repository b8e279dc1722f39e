"""Host <-> device helpers for the GPU tests (marshalling only)."""
import sys

import numpy as np
import pytest


def torch_cuda():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def to_dev(a: np.ndarray):
    """float32 -> float32 tensor; uint16 (bf16 bits) -> bfloat16 tensor."""
    import torch
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16).copy()).view(torch.bfloat16).cuda()
    return torch.from_numpy(a.copy()).cuda()


def to_host(t) -> np.ndarray:
    import torch
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def raw_to_dev(a: np.ndarray):
    """Any numpy array as a uint8 device tensor of the same bytes."""
    import torch
    return torch.from_numpy(np.ascontiguousarray(a).view(np.uint8).ravel().copy()).cuda()


def say(*args):
    print(*args, file=sys.stderr, flush=True)
