"""Fused linear log-prob / entropy, forward and backward, in float64 numpy.

TEST INFRASTRUCTURE ONLY -- see the package docstring.

The block-sparse tricks on the page (tile skipping, span-local dHidden, the
live-width final vocabulary split) only skip work whose contribution is exactly
zero, so the oracle is the plain dense, masked definition.  It follows:

* SkyRL #2376, "What does this PR do?" and the Bugbot "Overview": the LM-head
  projection is fused with the per-token target log-prob; the forward never
  materialises the [T, V] logits (here: only a block of token rows at a time).
* The stack's "fuse LM-head entropy for RL" layer and "Test coverage" (the
  entropy parity test keeps an independent fp64 reference): per-token entropy
  of the softmax over the vocabulary, with its gradient.
* The Gemini "Code Review" suggestion: the hidden gradient is the accumulated
  product of d-logits with the weight rows, ``d_hidden += d_logits @ weight``.
* "How it works": weight gradients stay a dense contraction over all tokens.

Definition (all arithmetic float64; inputs are the exact stored values widened):

    z[t, v]      = sum_k h[t, k] * W[v, k]
    lse[t]       = M + ln sum_v exp(z[t, v] - M),        M = max_v z[t, v]
    p[t, v]      = exp(z[t, v] - lse[t])
    logprob[t]   = z[t, y[t]] - lse[t]
    entropy[t]   = sum_v p[t, v] * (lse[t] - z[t, v])   (nats, temperature 1)
    ga, gb       = mask * grad_logprob, mask * grad_entropy   (None -> 0)
    Ez[t]        = sum_v p[t, v] * z[t, v]
    dz[t, v]     = ga[t] * ([v == y[t]] - p[t, v]) + gb[t] * p[t, v] * (Ez[t] - z[t, v])
    dH           = dz @ W          dW = dz^T @ h

The gradient of logprob w.r.t. z is (onehot - p); that of the entropy is
p * (Ez - z).  The pages do not print these; finite differences pin them.

Readings: targets lie in [0, V) (no ignore index; out of range raises); the
loss mask alone decides which tokens contribute (nonzero = active); an absent
upstream gradient is zero.
"""

from __future__ import annotations

from typing import Iterable, Tuple

import numpy as np


def widen_bf16(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> the exact float64 values they encode."""
    b = np.ascontiguousarray(bits).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def _check_targets(y: np.ndarray, V: int) -> np.ndarray:
    y = np.asarray(y, dtype=np.int64)
    if y.size and (y.min() < 0 or y.max() >= V):
        raise ValueError("targets must lie in [0, V)")
    return y


def _row_stats(z: np.ndarray, y: np.ndarray):
    """For a block of logit rows: lse, p, logprob, entropy, Ez (definition)."""
    M = z.max(axis=1)
    lse = M + np.log(np.exp(z - M[:, None]).sum(axis=1))
    p = np.exp(z - lse[:, None])
    zy = z[np.arange(z.shape[0]), y]
    logprob = zy - lse
    entropy = (p * (lse[:, None] - z)).sum(axis=1)
    Ez = (p * z).sum(axis=1)
    return lse, p, logprob, entropy, Ez


def forward(h, W, targets, block: int = 64) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Returns (logprob, entropy, lse), each float64 [T].

    h: [T, H], W: [V, H], targets: int [T] in [0, V)."""
    h = _f64(h)
    W = _f64(W)
    T = h.shape[0]
    V = W.shape[0]
    y = _check_targets(targets, V)
    lp = np.empty(T)
    ent = np.empty(T)
    lse = np.empty(T)
    for t0 in range(0, T, block):
        t1 = min(T, t0 + block)
        z = h[t0:t1] @ W.T
        l, _, a, b, _ = _row_stats(z, y[t0:t1])
        lse[t0:t1], lp[t0:t1], ent[t0:t1] = l, a, b
    return lp, ent, lse


def dlogits(z: np.ndarray, y: np.ndarray, ga: np.ndarray, gb: np.ndarray) -> np.ndarray:
    """d(loss)/d(z) for a block of logit rows, where the loss is
    sum_t ga[t] * logprob[t] + gb[t] * entropy[t] (definition above)."""
    _, p, _, _, Ez = _row_stats(z, y)
    onehot = np.zeros_like(z)
    onehot[np.arange(z.shape[0]), y] = 1.0
    return ga[:, None] * (onehot - p) + gb[:, None] * p * (Ez[:, None] - z)


def _upstream(T: int, loss_mask, g) -> np.ndarray:
    m = np.ones(T) if loss_mask is None else (np.asarray(loss_mask) != 0).astype(np.float64)
    if g is None:
        return np.zeros(T)
    return m * _f64(g)


def backward(h, W, targets, loss_mask, grad_logprob, grad_entropy,
             block: int = 64) -> Tuple[np.ndarray, np.ndarray]:
    """Returns (dH [T, H], dW [V, H]) in float64.

    loss_mask: [T] (nonzero = active) or None (all active).
    grad_logprob, grad_entropy: [T] or None (zero)."""
    h = _f64(h)
    W = _f64(W)
    T, H = h.shape
    V = W.shape[0]
    y = _check_targets(targets, V)
    ga = _upstream(T, loss_mask, grad_logprob)
    gb = _upstream(T, loss_mask, grad_entropy)
    dH = np.zeros((T, H))
    dW = np.zeros((V, H))
    for t0 in range(0, T, block):
        t1 = min(T, t0 + block)
        z = h[t0:t1] @ W.T
        dz = dlogits(z, y[t0:t1], ga[t0:t1], gb[t0:t1])
        dH[t0:t1] = dz @ W
        dW += dz.T @ h[t0:t1]
    return dH, dW


def forward_rows(h, W, targets, rows: Iterable[int]):
    """(logprob, entropy, lse) for selected tokens only; each token's outputs
    depend on its own hidden row alone, so this is exact at any T."""
    rows = np.asarray(list(rows), dtype=np.int64)
    h = _f64(np.asarray(h)[rows])
    y = np.asarray(targets)[rows]
    return forward(h, W, y)


def dhidden_rows(h, W, targets, loss_mask, grad_logprob, grad_entropy,
                 rows: Iterable[int]) -> np.ndarray:
    """dH rows for selected tokens only (each depends on its own token alone)."""
    rows = np.asarray(list(rows), dtype=np.int64)
    W = _f64(W)
    V = W.shape[0]
    hr = _f64(np.asarray(h)[rows])
    y = _check_targets(np.asarray(targets)[rows], V)
    m = None if loss_mask is None else np.asarray(loss_mask)[rows]
    ga = _upstream(len(rows), m, None if grad_logprob is None else np.asarray(grad_logprob)[rows])
    gb = _upstream(len(rows), m, None if grad_entropy is None else np.asarray(grad_entropy)[rows])
    z = hr @ W.T
    return dlogits(z, y, ga, gb) @ W


def loss(h, W, targets, loss_mask, grad_logprob, grad_entropy) -> float:
    """The scalar whose gradient backward() returns:
    L = sum_t m_t * (a_t * logprob_t + b_t * entropy_t).  Used by the
    finite-difference pin."""
    lp, ent, _ = forward(h, W, targets)
    T = lp.shape[0]
    return float((_upstream(T, loss_mask, grad_logprob) * lp).sum()
                 + (_upstream(T, loss_mask, grad_entropy) * ent).sum())

