"""flh_spans_build on the GPU, bit-exact against the span oracle.

Spans, span count, active count and the tile bitmap are integer results with a
unique answer (SkyRL #2376, Bugbot "Overview": runs of the loss mask coalesced
across gaps <= 128; "How it works": tiles without an active token are skipped),
so every comparison is exact equality.
"""

import itertools

import numpy as np
import pytest
import torch

from entropy_block_sparse_amd import flh_spans_build
from oracle import spans as S
from tests.gpu_common import announce, cuda_device
from tests.helpers import load_span_examples
from workloads import make_mask

pytestmark = pytest.mark.gpu


def check_one(mask_np, G, tile_m=128, dev=None):
    m = torch.as_tensor(np.asarray(mask_np, np.uint8)).to(dev)
    meta = flh_spans_build(m, max_gap=G, tile_m=tile_m)
    got_spans = meta.host_spans()
    want = S.active_spans(mask_np, G)
    assert got_spans == want, (G, len(mask_np))
    assert int(meta.active_count.item()) == S.active_count(mask_np)
    n_words = len(S.tile_bits(mask_np, tile_m))
    assert meta.host_bits()[:n_words] == S.tile_bits(mask_np, tile_m)


def test_all_masks_up_to_10_tokens():
    dev = cuda_device()
    announce("spans: all masks T<=10, G in {0,1,2,5}")
    for T in range(1, 11):
        for bits in itertools.product((0, 1), repeat=T):
            for G in (0, 1, 2, 5):
                check_one(list(bits), G, tile_m=3, dev=dev)


def test_worked_examples():
    dev = cuda_device()
    announce("spans: worked examples")
    for name, c in load_span_examples().items():
        for G in c["spans"]:
            for BM in (c["bits"] or {128: None}):
                check_one(c["mask"], G, tile_m=BM, dev=dev)


@pytest.mark.parametrize("T", [1, 63, 1023, 1024, 1025, 4097, 100003, 262144])
def test_random_masks(T):
    dev = cuda_device()
    rng = np.random.default_rng(T)
    for trial in range(4):
        p = [0.02, 0.3, 0.7, 0.98][trial]
        # bursty mask: runs with random lengths so gaps straddle the bound
        mask = np.zeros(T, np.uint8)
        t = 0
        on = bool(rng.random() < p)
        while t < T:
            n = int(rng.integers(1, 300))
            if on:
                mask[t:t + n] = 1
            t += n
            on = bool(rng.random() < p)
        for G in (0, 47, 128, 129):
            announce(f"spans: random T={T} p={p} G={G}")
            check_one(mask, G, dev=dev)


@pytest.mark.parametrize("cid,frac", [(1, None), (2, None), (3, None), (4, None),
                                      (5, 0.05), (5, 0.25), (5, 0.5), (5, 0.9), (5, 1.0)])
def test_workload_masks(cid, frac):
    dev = cuda_device()
    mask, _ = make_mask(cid, active_frac=frac)
    announce(f"spans: workload {cid} frac={frac}")
    check_one(mask, 128, dev=dev)


def test_edge_masks():
    dev = cuda_device()
    for T in (1, 2, 129, 5000):
        for fill in (0, 1):
            announce(f"spans: constant mask T={T} fill={fill}")
            check_one(np.full(T, fill, np.uint8), 128, dev=dev)
    # nonzero bytes other than 1 are active
    check_one(np.array([0, 7, 255, 0, 0, 3], np.uint8), 1, dev=dev)
