"""Pins for the fp64 LM-head oracle (CPU only).

Each pin is something other than the oracle's own formula:
* closed forms for one-hot-dominant logits (uniform logits give logprob = -ln V
  and entropy = ln V; a dominant logit d gives lse = ln(e^d + V - 1) and
  entropy = lse - d e^(d - lse), which tends to 0 as d grows), including the
  closed-form gradient of that case;
* independent library routines (scipy's logsumexp, log_softmax, softmax and
  entropy) on random logits;
* central finite differences of the oracle's own forward for dH and dW;
* invariants (d-logits rows sum to zero so sum_v dW[v] = 0; zero weights give
  zero dH; shift invariance; bounds; inactive tokens contribute nothing);
* a separate pure-Python rendering (``oracle.tiny``) on small shapes.
Planted mistakes (sign of the entropy term, dropped one-hot term, an off-by-one
target) are shown to fail these pins.

Sources: SkyRL #2376 "What does this PR do?" / Bugbot "Overview" (fused
linear log-prob), "Test coverage" (independent fp64 entropy reference,
gradients against dense references), Gemini "Code Review" (d_hidden
accumulates d_logits @ weight), "How it works" (dense weight gradient).
"""

import math

import numpy as np
import pytest
import scipy.special as sps
import scipy.stats as sst

from oracle import lmhead as O
from oracle import tiny


def one_hot_case(V, H, d, k, y):
    """h = e_0 for every token, W[k, 0] = d, all else 0 -> z[t] = d at v=k, 0 elsewhere."""
    T = len(y)
    h = np.zeros((T, H))
    h[:, 0] = 1.0
    W = np.zeros((V, H))
    W[k, 0] = d
    return h, W, np.asarray(y, np.int64)


LN_V = {  # ln V, 16 significant digits
    4096: 8.317766166719343,
    128256: 11.76178354556443,
    32064: 10.37548918444454,
    152064: 11.93205676384221,
    129280: 11.76973587375492,
}


@pytest.mark.parametrize("V", sorted(LN_V))
def test_uniform_logits_closed_form(V):
    h, W, y = one_hot_case(V, 8, 0.0, 3, [0, 3, V - 1])
    lp, ent, lse = O.forward(h, W, y)
    assert np.allclose(lp, -LN_V[V], rtol=0, atol=1e-12)
    assert np.allclose(ent, LN_V[V], rtol=0, atol=1e-12)
    assert np.allclose(lse, LN_V[V], rtol=0, atol=1e-12)
    assert abs(math.log(V) - LN_V[V]) < 1e-13


@pytest.mark.parametrize("d", [0.5, 4.0, 16.0, 30.0, -7.0])
def test_dominant_logit_closed_form(d):
    V, k = 4096, 17
    h, W, y = one_hot_case(V, 4, d, k, [k, 0, V - 1])
    lp, ent, lse = O.forward(h, W, y)
    L = math.log(math.exp(d) + V - 1)
    assert np.allclose(lse, L, rtol=1e-14, atol=0)
    assert abs(lp[0] - (d - L)) < 1e-12
    assert abs(lp[1] + L) < 1e-12 and abs(lp[2] + L) < 1e-12
    H_cf = L - d * math.exp(d - L)
    assert np.allclose(ent, H_cf, rtol=1e-9, atol=1e-13)


def test_dominant_logit_reference_values():
    # Closed-form numbers, V = 4096, d = 16: logprob of the dominant token -4.6072539e-4, entropy 7.83063375e-3;
    # d = 30: entropy 1.1879e-8 (the near one-hot limit, entropy -> 0).
    V, k = 4096, 5
    h, W, y = one_hot_case(V, 2, 16.0, k, [k])
    lp, ent, _ = O.forward(h, W, y)
    assert abs(lp[0] - (-4.6072539e-4)) < 1e-11
    assert abs(ent[0] - 7.83063375e-3) < 1e-11
    h, W, y = one_hot_case(V, 2, 30.0, k, [k])
    _, ent, _ = O.forward(h, W, y)
    assert abs(ent[0] - 1.1879e-8) < 1e-12


def test_dominant_logit_gradient_closed_form():
    V, H, k, d, a = 11, 3, 4, 2.5, 0.7
    h, W, y = one_hot_case(V, H, d, k, [k, 2])
    mask = np.array([1, 1], np.uint8)
    ga = np.array([a, a])
    dH, dW = O.backward(h, W, y, mask, ga, None)
    Z = math.exp(d) + V - 1
    pk, pj = math.exp(d) / Z, 1.0 / Z
    # token 0 (target k): dz_k = a(1 - pk), dz_j = -a pj; dH[0, 0] = d * dz_k
    assert abs(dH[0, 0] - d * a * (1 - pk)) < 1e-14
    # token 1 (target 2): dz_k = -a pk -> dH[1, 0] = -d a pk
    assert abs(dH[1, 0] - (-d * a * pk)) < 1e-14
    assert np.all(dH[:, 1:] == 0.0)
    # dW[v, 0] = sum_t dz[t, v] (h = e_0)
    want = np.full(V, -2 * a * pj)
    want[k] = a * (1 - pk) - a * pk
    want[2] = -a * pj + a * (1 - pj)
    assert np.allclose(dW[:, 0], want, atol=1e-14, rtol=0)
    assert np.all(dW[:, 1:] == 0.0)


def _random_case(rng, T, H, V, scale=1.0):
    h = rng.normal(size=(T, H)) * scale
    W = rng.normal(size=(V, H)) * scale
    y = rng.integers(0, V, T)
    return h, W, y


def test_forward_matches_scipy_routines():
    rng = np.random.default_rng(3)
    h, W, y = _random_case(rng, 37, 24, 301, 0.7)
    lp, ent, lse = O.forward(h, W, y, block=8)
    z = np.einsum("tk,vk->tv", h, W)
    assert np.allclose(lse, sps.logsumexp(z, axis=1), rtol=1e-13, atol=1e-13)
    assert np.allclose(lp, sps.log_softmax(z, axis=1)[np.arange(37), y], rtol=1e-12, atol=1e-12)
    assert np.allclose(ent, sst.entropy(sps.softmax(z, axis=1), axis=1), rtol=1e-11, atol=1e-12)


def test_forward_block_size_independent():
    rng = np.random.default_rng(4)
    h, W, y = _random_case(rng, 50, 16, 97)
    a = O.forward(h, W, y, block=1)
    b = O.forward(h, W, y, block=64)
    for x, z in zip(a, b):
        assert np.allclose(x, z, rtol=1e-14, atol=1e-14)


def _fd_grads(h, W, y, mask, a, b, eps=1e-6):
    def L(hh, WW):
        return O.loss(hh, WW, y, mask, a, b)
    gH = np.zeros_like(h)
    for i in np.ndindex(h.shape):
        hp, hm = h.copy(), h.copy()
        hp[i] += eps
        hm[i] -= eps
        gH[i] = (L(hp, W) - L(hm, W)) / (2 * eps)
    gW = np.zeros_like(W)
    for i in np.ndindex(W.shape):
        Wp, Wm = W.copy(), W.copy()
        Wp[i] += eps
        Wm[i] -= eps
        gW[i] = (L(h, Wp) - L(h, Wm)) / (2 * eps)
    return gH, gW


def _fd_error(backward_fn, seed=5, mode="both"):
    rng = np.random.default_rng(seed)
    T, H, V = 7, 5, 11
    h, W, y = _random_case(rng, T, H, V, 0.8)
    mask = np.array([1, 0, 1, 1, 0, 1, 1], np.uint8)
    a = rng.uniform(-1, 1, T)
    b = rng.uniform(-1, 1, T) if mode == "both" else None
    dH, dW = backward_fn(h, W, y, mask, a, b)
    gH, gW = _fd_grads(h, W, y, mask, a, b)
    e1 = np.max(np.abs(dH - gH)) / max(1e-30, np.max(np.abs(gH)))
    e2 = np.max(np.abs(dW - gW)) / max(1e-30, np.max(np.abs(gW)))
    return max(e1, e2)


@pytest.mark.parametrize("mode", ["both", "lp"])
def test_backward_matches_finite_differences(mode):
    assert _fd_error(O.backward, mode=mode) < 1e-6


def test_backward_invariants():
    rng = np.random.default_rng(6)
    T, H, V = 40, 12, 57
    h, W, y = _random_case(rng, T, H, V)
    mask = (rng.random(T) < 0.6).astype(np.uint8)
    a = rng.uniform(-1, 1, T)
    b = rng.uniform(-1, 1, T)
    dH, dW = O.backward(h, W, y, mask, a, b, block=16)
    # d-logits rows sum to zero -> sum over vocab rows of dW vanishes
    assert np.max(np.abs(dW.sum(axis=0))) < 1e-12 * max(1.0, np.abs(dW).max()) * V
    # inactive tokens: exactly zero hidden gradient
    assert np.all(dH[mask == 0] == 0.0)
    # masking the upstream gradients by hand changes nothing
    dH2, dW2 = O.backward(h, W, y, None, a * mask, b * mask, block=16)
    assert np.allclose(dH, dH2, rtol=0, atol=1e-15) and np.allclose(dW, dW2, rtol=0, atol=1e-15)
    # zero weights -> zero hidden gradient
    dH0, _ = O.backward(h, np.zeros_like(W), y, mask, a, b)
    assert np.all(dH0 == 0.0)
    # uniform logits with entropy-only upstream -> zero d-logits
    dHu, dWu = O.backward(h, np.zeros_like(W), y, mask, None, b)
    assert np.all(dHu == 0.0) and np.all(dWu == 0.0)


def test_shift_invariance_and_bounds():
    rng = np.random.default_rng(8)
    T, H, V = 30, 9, 64
    h, W, y = _random_case(rng, T, H, V)
    c = rng.normal(size=H)
    lp, ent, _ = O.forward(h, W, y)
    lp2, ent2, _ = O.forward(h, W + c[None, :], y)
    assert np.allclose(lp, lp2, atol=1e-11) and np.allclose(ent, ent2, atol=1e-11)
    assert np.all(lp <= 0) and np.all(ent >= -1e-15) and np.all(ent <= math.log(V) + 1e-12)
    mask = np.ones(T, np.uint8)
    a = rng.uniform(-1, 1, T)
    b = rng.uniform(-1, 1, T)
    dH, dW = O.backward(h, W, y, mask, a, b)
    dH2, dW2 = O.backward(h, W + c[None, :], y, mask, a, b)
    assert np.allclose(dH, dH2, atol=1e-10) and np.allclose(dW, dW2, atol=1e-10)


def test_row_helpers_match_full():
    rng = np.random.default_rng(9)
    T, H, V = 33, 8, 70
    h, W, y = _random_case(rng, T, H, V)
    mask = (rng.random(T) < 0.5).astype(np.uint8)
    a = rng.uniform(-1, 1, T)
    b = rng.uniform(-1, 1, T)
    rows = [0, 5, 17, 32]
    lp, ent, lse = O.forward(h, W, y)
    rlp, rent, rlse = O.forward_rows(h, W, y, rows)
    assert np.allclose(rlp, lp[rows], atol=1e-14) and np.allclose(rent, ent[rows], atol=1e-14)
    dH, _ = O.backward(h, W, y, mask, a, b)
    assert np.allclose(O.dhidden_rows(h, W, y, mask, a, b, rows), dH[rows], atol=1e-14)


def test_targets_out_of_range_raise():
    h = np.ones((2, 3))
    W = np.ones((4, 3))
    with pytest.raises(ValueError):
        O.forward(h, W, [0, 4])
    with pytest.raises(ValueError):
        O.forward(h, W, [-1, 0])


def test_widen_bf16_exact():
    bits = np.array([0x3F80, 0xBF80, 0x0000, 0x3FC0, 0x4049, 0x0001], np.uint16)
    want = [1.0, -1.0, 0.0, 1.5, 3.140625, 2.0 ** -133]
    assert list(O.widen_bf16(bits)) == want


def test_tiny_python_matches_numpy():
    rng = np.random.default_rng(10)
    for T, H, V in [(1, 1, 2), (3, 4, 5), (6, 7, 13), (9, 3, 16)]:
        h, W, y = _random_case(rng, T, H, V)
        mask = (rng.random(T) < 0.7).astype(np.uint8)
        a = rng.uniform(-1, 1, T)
        b = rng.uniform(-1, 1, T)
        lp, ent, lse = O.forward(h, W, y)
        tlp, tent, tlse = tiny.forward(h.tolist(), W.tolist(), y.tolist())
        assert np.allclose(lp, tlp, atol=1e-12) and np.allclose(ent, tent, atol=1e-12)
        dH, dW = O.backward(h, W, y, mask, a, b)
        tdH, tdW = tiny.backward(h.tolist(), W.tolist(), y.tolist(), mask.tolist(), a.tolist(), b.tolist())
        assert np.allclose(dH, tdH, atol=1e-12) and np.allclose(dW, tdW, atol=1e-12)


# ---- planted mistakes: each must be caught by one of the pins above ----------

def _planted_backward(variant):
    def dl(z, y, ga, gb):
        _, p, _, _, Ez = O._row_stats(z, y)
        onehot = np.zeros_like(z)
        if variant == "target_off_by_one":
            onehot[np.arange(z.shape[0]), (y + 1) % z.shape[1]] = 1.0
        else:
            onehot[np.arange(z.shape[0]), y] = 1.0
        if variant == "entropy_sign":
            return ga[:, None] * (onehot - p) + gb[:, None] * p * (z - Ez[:, None])
        if variant == "drop_onehot":
            return ga[:, None] * (-p) + gb[:, None] * p * (Ez[:, None] - z)
        return ga[:, None] * (onehot - p) + gb[:, None] * p * (Ez[:, None] - z)

    def bw(h, W, y, mask, a, b):
        saved = O.dlogits
        O.dlogits = dl
        try:
            return O.backward(h, W, y, mask, a, b)
        finally:
            O.dlogits = saved
    return bw


@pytest.mark.parametrize("variant", ["entropy_sign", "drop_onehot", "target_off_by_one"])
def test_planted_backward_mistakes_are_caught(variant):
    assert _fd_error(_planted_backward(variant)) > 1e-2


def test_planted_span_mistakes_are_caught():
    from oracle import spans as S
    from tests.test_oracle_spans import characterize

    def strict_gap(mask, G):  # '<' instead of '<=' when merging
        out = []
        for s, e in S.active_runs(mask):
            if out and s - out[-1][1] < G:
                out[-1] = (out[-1][0], e)
            else:
                out.append((s, e))
        return out

    def end_off_by_one(mask, G):
        return [(s, e - 1) if e - s > 1 else (s, e) for s, e in S.active_spans(mask, G)]

    mask = [1, 1, 0, 0, 1, 1, 1, 0, 1]
    for bad in (strict_gap, end_off_by_one):
        with pytest.raises(AssertionError):
            characterize(mask, 2, bad(mask, 2))
