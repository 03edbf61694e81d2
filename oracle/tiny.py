"""The fused linear log-prob / entropy definition in pure Python loops.

TEST INFRASTRUCTURE ONLY -- see the package docstring.

Same definition as :mod:`oracle.lmhead` (SkyRL #2376, "What does this PR do?",
Bugbot "Overview", "Test coverage"), written element by element with exactly
rounded sums (``math.fsum``).  It is meant for a handful of tokens, hidden
units and vocabulary rows (say <= 16 each); it cross-checks the numpy version,
which uses BLAS for its products.
"""

from __future__ import annotations

import math
from typing import List, Optional, Sequence, Tuple

Mat = List[List[float]]


def logits(h: Mat, W: Mat) -> Mat:
    return [[math.fsum(hk * wk for hk, wk in zip(ht, wv)) for wv in W] for ht in h]


def forward(h: Mat, W: Mat, y: Sequence[int]) -> Tuple[List[float], List[float], List[float]]:
    """Returns (logprob, entropy, lse) as lists."""
    V = len(W)
    z = logits(h, W)
    lp, ent, lse = [], [], []
    for t, row in enumerate(z):
        if not 0 <= y[t] < V:
            raise ValueError("target out of range")
        M = max(row)
        l = M + math.log(math.fsum(math.exp(v - M) for v in row))
        p = [math.exp(v - l) for v in row]
        lse.append(l)
        lp.append(row[y[t]] - l)
        ent.append(math.fsum(pv * (l - v) for pv, v in zip(p, row)))
    return lp, ent, lse


def backward(h: Mat, W: Mat, y: Sequence[int], mask: Optional[Sequence[int]],
             ga: Optional[Sequence[float]], gb: Optional[Sequence[float]]) -> Tuple[Mat, Mat]:
    """Returns (dH, dW) as nested lists; absent grads are zero, absent mask is
    all-active, inactive tokens contribute nothing."""
    T, H, V = len(h), len(h[0]), len(W)
    z = logits(h, W)
    dz: Mat = []
    for t in range(T):
        act = 1.0 if (mask is None or mask[t]) else 0.0
        a = act * (ga[t] if ga is not None else 0.0)
        b = act * (gb[t] if gb is not None else 0.0)
        row = z[t]
        M = max(row)
        l = M + math.log(math.fsum(math.exp(v - M) for v in row))
        p = [math.exp(v - l) for v in row]
        ez = math.fsum(pv * v for pv, v in zip(p, row))
        dz.append([a * ((1.0 if v == y[t] else 0.0) - p[v]) + b * p[v] * (ez - row[v])
                   for v in range(V)])
    dH = [[math.fsum(dz[t][v] * W[v][k] for v in range(V)) for k in range(H)] for t in range(T)]
    dW = [[math.fsum(dz[t][v] * h[t][k] for t in range(T)) for k in range(H)] for v in range(V)]
    return dH, dW
