"""flh_forward_noalloc (the forward with its scratch in a static device array, for
callers that cannot allocate) against flh_forward_ex, the entry point it is a variant
of: the same kernels on the same inputs, so the outputs must be equal bitwise.  Two
calls in a row, the second smaller, so the second reads an array that still holds the
first call's contents; both the dense forward and the forward over active tiles."""

import ctypes

import numpy as np
import pytest
import torch

from entropy_block_sparse_amd import flh_forward, flh_spans_build
from entropy_block_sparse_amd._lib import FLH_BF16, FLH_F32, FLH_FWD_SKIP_INACTIVE, check, lib
from tests.gpu_common import announce, cuda_device
from workloads import make_tensors

pytestmark = pytest.mark.gpu


def _noalloc(h, W, y, meta=None, flags=0):
    T, H = h.shape
    V = W.shape[0]
    out = [torch.empty(T, dtype=torch.float32, device=h.device) for _ in range(3)]
    st = ctypes.c_void_p(torch.cuda.current_stream(h.device).cuda_stream)
    dt = FLH_BF16 if h.dtype == torch.bfloat16 else FLH_F32
    mp = ctypes.byref(meta.struct) if meta is not None else None
    check(lib().flh_forward_noalloc(dt, ctypes.c_void_p(h.data_ptr()), ctypes.c_void_p(W.data_ptr()),
                                    ctypes.c_void_p(y.data_ptr()), T, H, V,
                                    *[ctypes.c_void_p(o.data_ptr()) for o in out], mp, st, flags),
          "flh_forward_noalloc")
    return out


def _mask(T, seed):
    rng = np.random.default_rng(seed)
    m = np.zeros(T, np.uint8)
    for _ in range(6):
        s = int(rng.integers(0, T))
        m[s:s + int(rng.integers(1, 400))] = 1
    return m


@pytest.mark.parametrize("dtype,skip", [("bf16", False), ("bf16", True), ("f32", False)])
def test_noalloc_forward_equals_forward_ex_on_two_calls(dtype, skip):
    dev = cuda_device()
    for k, (T, H, V) in enumerate([(4000, 512, 30000), (900, 256, 5000)]):
        announce(f"noalloc forward call {k}: T={T} H={H} V={V} {dtype} skip={skip}")
        h, W, y = [x.to(dev) for x in make_tensors(T, H, V, dtype, 80 + k)]
        meta = flh_spans_build(torch.as_tensor(_mask(T, 90 + k)).to(dev)) if skip else None
        ref = flh_forward(h, W, y, meta=meta, skip_inactive=skip)
        got = _noalloc(h, W, y, meta, FLH_FWD_SKIP_INACTIVE if skip else 0)
        torch.cuda.synchronize()
        for r, g in zip(ref, got):
            assert torch.equal(r, g)


def test_noalloc_forward_at_the_largest_llama_shape():
    """T = 16384 at V = 128256 needs about 125 MiB of the 128 MiB scratch."""
    dev = cuda_device()
    T, H, V = 16384, 512, 128256
    announce(f"noalloc forward at the scratch limit T={T} H={H} V={V}")
    h, W, y = [x.to(dev) for x in make_tensors(T, H, V, "bf16", 99)]
    ref = flh_forward(h, W, y)
    got = _noalloc(h, W, y)
    torch.cuda.synchronize()
    for r, g in zip(ref, got):
        assert torch.equal(r, g)
