"""Test-side widening of stored inputs to fp64 through PyTorch's own dtype
conversions, independent of the oracle's bit manipulation: the pins that
compare the oracle with brute force or with PyTorch's attention read their
inputs through this module, so a mistake in the oracle's widening (a wrong
shift, a lost sign) cannot cancel out of the comparison.
"""

import numpy as np
import torch

import workloads as W


def torch_to_f64(arr, dtype):
    """Stored data (float32, or uint16 bf16 patterns) -> float64 via torch."""
    a = np.ascontiguousarray(arr)
    if dtype == W.F32:
        assert a.dtype == np.float32
        return torch.from_numpy(a).to(torch.float64).numpy()
    if dtype == W.BF16:
        assert a.dtype == np.uint16
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    raise ValueError(dtype)
