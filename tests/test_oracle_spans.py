"""Pins for the span / tile-bitmap oracle (CPU only).

The oracle builds spans by scanning runs and merging; these tests never use
that construction.  They check its output against a characterisation that
determines the span list uniquely (brute force over every mask of up to 12
tokens, and all 14-token masks at one gap bound), against hand-derived worked
examples (tests/golden/spans_worked_examples.txt), and against the capacity
bound.  Rule: SkyRL #2376, Bugbot "Overview" (runs of active tokens coalesced
across gaps of at most 128) and "How it works" (ordered spans, no token
reordering; only active d-logits tiles are processed).
"""

import itertools

import numpy as np
import pytest

from oracle import spans as S
from tests.helpers import load_span_examples


def characterize(mask, G, spans):
    """Assert the conditions that fix the span list:
    (i)   every active token lies in exactly one span;
    (ii)  every span starts and ends on an active token;
    (iii) spans are non-empty, inside [0, T), sorted and disjoint;
    (iv)  consecutive spans are separated by more than G tokens;
    (v)   inside a span every maximal inactive run has at most G tokens.
    Two consecutive active tokens share a span iff the inactive run between
    them is <= G: (iv) forbids splitting such a pair, (v) forbids joining a
    farther pair, so (i)-(v) admit exactly one span list."""
    T = len(mask)
    cover = [0] * T
    for s, e in spans:
        assert 0 <= s < e <= T
        assert mask[s] and mask[e - 1]
        for t in range(s, e):
            cover[t] += 1
    for t in range(T):
        if mask[t]:
            assert cover[t] == 1
        else:
            assert cover[t] <= 1
    for (s0, e0), (s1, e1) in zip(spans, spans[1:]):
        assert e0 < s1
        assert s1 - e0 > G
    for s, e in spans:
        run = 0
        for t in range(s, e):
            run = run + 1 if not mask[t] else 0
            assert run <= G


@pytest.mark.parametrize("G", [0, 1, 2, 3, 5])
def test_brute_force_all_masks_up_to_12(G):
    for T in range(0, 13):
        for bits in itertools.product((0, 1), repeat=T):
            sp = S.active_spans(bits, G)
            characterize(bits, G, sp)
            assert S.active_count(bits) == sum(bits)


def test_brute_force_all_masks_14_gap2():
    for bits in itertools.product((0, 1), repeat=14):
        characterize(bits, 2, S.active_spans(bits, 2))


@pytest.mark.parametrize("G", [0, 1, 2, 3])
def test_capacity_is_the_maximum(G):
    for T in range(1, 13):
        best = max(len(S.active_spans(b, G)) for b in itertools.product((0, 1), repeat=T))
        assert best == S.span_capacity(T, G)


def test_capacity_examples():
    assert S.span_capacity(16384, 128) == 127
    assert S.span_capacity(262144, 128) == 2017
    assert S.span_capacity(0, 128) == 0


def test_tile_bits_against_token_to_tile_map():
    rng = np.random.default_rng(7)
    for _ in range(200):
        T = int(rng.integers(1, 300))
        BM = int(rng.choice([1, 3, 32, 64, 128]))
        mask = (rng.random(T) < rng.random() * 0.3).astype(np.uint8)
        words = S.tile_bits(mask, BM)
        n_tiles = -(-T // BM)
        assert len(words) == -(-n_tiles // 32)
        want = set(int(t) // BM for t in np.nonzero(mask)[0])
        got = {w * 32 + b for w, word in enumerate(words) for b in range(32) if (word >> b) & 1}
        assert got == want


def test_random_masks_large_G_variety():
    rng = np.random.default_rng(11)
    for _ in range(100):
        T = int(rng.integers(1, 600))
        G = int(rng.choice([0, 1, 47, 48, 128, 1000]))
        mask = (rng.random(T) < rng.random()).astype(np.uint8)
        characterize(list(mask), G, S.active_spans(mask, G))


def test_worked_examples():
    cases = load_span_examples()
    assert cases
    for name, c in cases.items():
        m = c["mask"]
        for G, want in c["spans"].items():
            assert S.active_spans(m, G) == want, (name, G)
        for BM, want in c["bits"].items():
            assert S.tile_bits(m, BM) == want, (name, BM)
        assert S.active_count(m) == c["count"], name


def test_span_tiles_partition_spans():
    sp = [(3, 10), (200, 713), (900, 901)]
    tiles = S.span_tiles(sp, 256)
    assert tiles == [(3, 10), (200, 456), (456, 712), (712, 713), (900, 901)]


def test_nonzero_bytes_are_active():
    assert S.active_spans([0, 2, 255, 0, 0, 9], 1) == [(1, 3), (5, 6)]
    assert S.active_count([0, 2, 255, 0, 0, 9]) == 3
