"""Calls on different streams, and from different host threads, run concurrently and give
the results they give alone, bitwise.

The library keeps no device state between calls (every buffer is the caller's; only the
no-allocation forward has a static scratch array, documented as racing) and its host state
is per thread (the tracer) or atomic (the compute-unit count).  Two different steps -- a
bf16 one and an fp8 one, different sizes -- run one after the other on the default stream
for the references, then at the same time on two streams (default priority), then from two
host threads with a stream each.
"""

import threading

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


def _case(kind, dev):
    if kind == "bf16":
        T, H, V, split, seed = 1000, 256, 3000, 1024, 61
        h, W, y = [x.to(dev) for x in make_tensors(T, H, V, "bf16", seed)]
    else:
        T, H, V, split, seed = 777, 128, 2600, 1024, 62
        hc, s_h, Wc, s_w, y = make_tensors_fp8(T, H, V, seed, device=dev)
    mask = _mask(T, seed)
    a, b = make_upstream(mask)
    m = torch.as_tensor(mask).to(dev)
    g_lp, g_ent = torch.as_tensor(a).to(dev), torch.as_tensor(b).to(dev)

    def step():
        meta = flh_spans_build(m)
        if kind == "bf16":
            lp, ent, lse = flh_forward(h, W, y)
            dH, dW = flh_backward(h, W, y, lse, ent, g_lp, g_ent, m, meta, split)
        else:
            lp, ent, lse = flh_forward_fp8(hc, s_h, Wc, s_w, y)
            dH, dW = flh_backward_fp8(hc, s_h, Wc, s_w, y, lse, ent, g_lp, g_ent, m, meta, split)
        return lp, ent, lse, dH, dW
    return step


def _same(ref, out, what):
    for name, r, x in zip(("logprob", "entropy", "lse", "dH", "dW"), ref, out):
        assert torch.equal(r, x), f"{what}: {name}"


def test_two_streams_and_two_threads_match_sequential():
    dev = cuda_device()
    announce("concurrency: bf16 and fp8 steps on two streams, then from two host threads")
    steps = [_case("bf16", dev), _case("fp8", dev)]
    refs = [[t.clone() for t in s()] for s in steps]
    torch.cuda.synchronize()

    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for s in streams:
        s.wait_stream(torch.cuda.current_stream())
    for it in range(3):
        outs = [None, None]
        for i in (0, 1):
            with torch.cuda.stream(streams[i]):
                outs[i] = steps[i]()
        torch.cuda.synchronize()
        for i in (0, 1):
            _same(refs[i], outs[i], f"two streams, pass {it}, step {i}")

    results, errors = [None, None], []

    def worker(i):
        try:
            torch.cuda.set_device(dev)
            with torch.cuda.stream(streams[i]):
                rs = [steps[i]() for _ in range(3)]
            streams[i].synchronize()
            results[i] = rs
        except Exception as e:  # reported below, on the main thread
            errors.append(repr(e))

    threads = [threading.Thread(target=worker, args=(i,)) for i in (0, 1)]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads), "a worker thread did not finish"
    assert not errors, errors
    torch.cuda.synchronize()
    for i in (0, 1):
        for k, out in enumerate(results[i]):
            _same(refs[i], out, f"thread {i}, call {k}")
