"""A whole step (metadata, forward, backward) captured into one HIP graph.

The library only enqueues kernels on the caller's stream -- no allocation, no memset,
no host synchronisation -- so a training step can be captured once and replayed.  The
graph is replayed several times with the program's own eager work and
synchronisations in between, and every replay must reproduce the eager outputs
bitwise (the kernels are deterministic).  Covered for the default path and for the
forward and weight gradient over active token tiles only, on bf16 and on fp8 (E4M3) inputs.
"""

import numpy as np
import pytest
import torch

from entropy_block_sparse_amd import flh_backward, flh_backward_fp8, flh_forward, flh_forward_fp8, flh_spans_build
from tests.gpu_common import announce, cuda_device
from workloads import make_tensors, make_tensors_fp8, make_upstream

pytestmark = pytest.mark.gpu


def _mask(T, seed):
    rng = np.random.default_rng(seed)
    m = np.zeros(T, np.uint8)
    t = 0
    while t < T:
        n = int(rng.integers(1, 300))
        if rng.random() < 0.5:
            m[t:t + n] = 1
        t += n
    return m


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
@pytest.mark.parametrize("skip", [False, True])
def test_captured_step_replays_match_eager(skip, dtype):
    dev = cuda_device()
    T, H, V, split = 1000, 256, 3000, 1024
    announce(f"graph capture T={T} H={H} V={V} skip={skip} dtype={dtype}")
    if dtype == "fp8":
        hc, s_h, Wc, s_w, y = make_tensors_fp8(T, H, V, 41, device=dev)
    else:
        h, W, y = [x.to(dev) for x in make_tensors(T, H, V, "bf16", 41)]
    mask_np = _mask(T, 42)
    a, b = make_upstream(mask_np)
    m = torch.as_tensor(mask_np).to(dev)
    g_lp, g_ent = torch.as_tensor(a).to(dev), torch.as_tensor(b).to(dev)

    def step():
        meta = flh_spans_build(m)
        if dtype == "fp8":
            lp, ent, lse = flh_forward_fp8(hc, s_h, Wc, s_w, y, meta=meta, skip_inactive=skip)
            dH, dW = flh_backward_fp8(hc, s_h, Wc, s_w, y, lse, ent, g_lp, g_ent, m, meta, split,
                                      skip_inactive_dw=skip)
        else:
            lp, ent, lse = flh_forward(h, W, y, meta=meta, skip_inactive=skip)
            dH, dW = flh_backward(h, W, y, lse, ent, g_lp, g_ent, m, meta, split, skip_inactive_dw=skip)
        return lp, ent, lse, dH, dW

    ref = [x.clone() for x in step()]
    torch.cuda.synchronize()

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()  # warm-up on a side stream before capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        out = step()
    torch.cuda.synchronize()

    for it in range(3):
        # the program's own eager work between replays, including this library's
        eager = step()
        junk = torch.randn(1 << 20, device=dev).mul_(3.0).sum()
        torch.cuda.synchronize()
        for x in out:  # poison the graph's outputs so a replay that skips a write is seen
            x.view(torch.uint8).fill_(0xFF)
        graph.replay()
        torch.cuda.synchronize()
        for name, r, x, e in zip(("logprob", "entropy", "lse", "dH", "dW"), ref, out, eager):
            assert torch.equal(r, x), f"replay {it}: {name}"
            assert torch.equal(r, e), f"eager {it}: {name}"
        del eager, junk
