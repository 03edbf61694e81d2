"""Helpers shared by the GPU tests: device fixture inputs and host copies.

Inputs come from the seeded generators in ``workloads``; expected values come
from ``oracle`` only.  Nothing here computes any part of the method.
"""

import numpy as np
import pytest
import torch


def cuda_device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def host64(t: torch.Tensor) -> np.ndarray:
    """Exact float64 copy of a bf16/fp32 device tensor (bf16 c fp32 c fp64)."""
    return t.detach().float().cpu().numpy().astype(np.float64)


def announce(msg: str) -> None:
    print(f"[gpu-case] {msg}", flush=True)


def dev_tensor(x, dev, dtype=None):
    t = torch.as_tensor(np.ascontiguousarray(x))
    if dtype is not None:
        t = t.to(dtype)
    return t.to(dev)
