"""Active-token metadata, by definition (pure Python).

TEST INFRASTRUCTURE ONLY -- see the package docstring.

What it follows:

* SkyRL #2376, "How it works": one builder derives the forward active mask and
  the backward spans from the token layout; the backward only touches active
  d-logits tiles; the hidden-gradient projection runs over the spans "without
  reordering tokens", i.e. spans are ordered and in token coordinates.
* SkyRL #2376, Bugbot "Overview": spans are runs of active tokens (from the RL
  loss mask) coalesced across gaps of at most 128 tokens.

Readings where the pages are silent:

* A token is active iff its loss-mask byte is nonzero.
* The gap between two runs is the number of inactive tokens strictly between
  them; two consecutive runs merge iff that gap is <= ``max_gap`` (inclusive).
* Spans are half-open ``(start, end)`` pairs in flat packed token coordinates,
  ascending and disjoint; they start and end on active tokens, so leading and
  trailing inactive tokens belong to no span.  Sequence boundaries of the packed
  row are not seen (the builder only sees the mask).
* Tile ``i`` of the bitmap covers tokens ``[i*tile_m, min(T, (i+1)*tile_m))``
  and is set iff any of them is active; bit ``i`` lives in 32-bit word
  ``i // 32`` at bit position ``i % 32`` (least significant first); unused bits
  of the last word are zero.
"""

from __future__ import annotations

from typing import List, Sequence, Tuple

Span = Tuple[int, int]


def _as_list(mask: Sequence[int]) -> List[int]:
    return [1 if int(x) != 0 else 0 for x in mask]


def active_count(mask: Sequence[int]) -> int:
    """Number of active tokens, A = sum of the mask (nonzero = active)."""
    return sum(_as_list(mask))


def active_runs(mask: Sequence[int]) -> List[Span]:
    """Maximal runs of consecutive active tokens, as half-open pairs, in order."""
    m = _as_list(mask)
    runs: List[Span] = []
    t = 0
    n = len(m)
    while t < n:
        if m[t]:
            s = t
            while t < n and m[t]:
                t += 1
            runs.append((s, t))
        else:
            t += 1
    return runs


def active_spans(mask: Sequence[int], max_gap: int = 128) -> List[Span]:
    """Ordered active spans: maximal active runs, consecutive runs merged when
    the number of inactive tokens between them is <= ``max_gap``
    (SkyRL #2376, Bugbot "Overview": "coalesced active spans (gaps <= 128)")."""
    if max_gap < 0:
        raise ValueError("max_gap must be >= 0")
    spans: List[Span] = []
    for s, e in active_runs(mask):
        if spans and s - spans[-1][1] <= max_gap:
            spans[-1] = (spans[-1][0], e)
        else:
            spans.append((s, e))
    return spans


def span_capacity(T: int, max_gap: int) -> int:
    """Largest possible number of spans for T tokens: n spans of >= 1 token need
    n + (n - 1) * (max_gap + 1) <= T tokens, so n <= (T + G + 1) // (G + 2)."""
    if T <= 0:
        return 0
    return (T + max_gap + 1) // (max_gap + 2)


def tile_flags(mask: Sequence[int], tile_m: int) -> List[int]:
    """One flag per token tile of height ``tile_m``: OR of the mask over the tile
    (SkyRL #2376, "How it works": only active d-logits tiles are processed)."""
    if tile_m <= 0:
        raise ValueError("tile_m must be positive")
    m = _as_list(mask)
    T = len(m)
    n_tiles = (T + tile_m - 1) // tile_m
    return [1 if any(m[i * tile_m:min(T, (i + 1) * tile_m)]) else 0 for i in range(n_tiles)]


def tile_bits(mask: Sequence[int], tile_m: int) -> List[int]:
    """The tile flags packed into uint32 words, least significant bit first."""
    flags = tile_flags(mask, tile_m)
    n_words = (len(flags) + 31) // 32
    words = [0] * n_words
    for i, f in enumerate(flags):
        if f:
            words[i // 32] |= 1 << (i % 32)
    return words


def span_tiles(spans: Sequence[Span], tile_rows: int) -> List[Span]:
    """Spans cut into row blocks of at most ``tile_rows`` tokens, each block
    starting at its span's start (span-local blocks; no token reordering)."""
    out: List[Span] = []
    for s, e in spans:
        r = s
        while r < e:
            out.append((r, min(e, r + tile_rows)))
            r += tile_rows
    return out
