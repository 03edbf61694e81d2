"""Pins of the FP8 (OCP E4M3) part of the oracle (CPU only).

* Every one of the 256 codes decodes to torch's float8_e4m3fn value (a library
  routine written independently of the oracle), NaNs in the same places.
* The values the format's definition fixes (tests/golden/e4m3_values.txt: zero, the
  subnormal and normal extremes, 448, NaN) come out exactly.
* Positive codes 0x00..0x7e are strictly increasing, and code c + 0x80 is -value(c).
* Every finite value is exactly a bfloat16 (so widening codes to bf16 loses nothing).
* The forward on codes reaches the closed forms of oracle.lmhead's pins through the
  scales: all-zero W codes give logprob = -ln V and entropy = ln V; one dominant logit
  d = scale_h * scale_w * value * value gives lse = ln(e^d + V - 1) and
  entropy = lse - d e^(d - lse), for scales that differ (a scale applied twice or to
  the wrong tensor fails).
"""

import math
import os

import numpy as np
import pytest
import torch

from oracle import fp8 as F

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "e4m3_values.txt")


def check_codes(decode):
    codes = np.arange(256, dtype=np.uint8)
    ours = decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    fin = ~np.isnan(ref)
    assert np.array_equal(ours[fin], ref[fin])
    assert np.array_equal(np.signbit(ours[fin]), np.signbit(ref[fin]))


def test_all_codes_match_torch_float8_e4m3fn():
    check_codes(F.decode_e4m3)


def test_values_the_definition_fixes():
    for line in open(GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        code, val = line.split()
        got = float(F.decode_e4m3(np.array([int(code, 16)], np.uint8))[0])
        if val == "nan":
            assert math.isnan(got), code
        else:
            assert got == float(val) and math.copysign(1.0, got) == math.copysign(1.0, float(val)), (code, got)


def test_order_sign_and_bf16_exactness():
    pos = F.decode_e4m3(np.arange(0x7f, dtype=np.uint8))
    assert np.all(np.diff(pos) > 0)
    neg = F.decode_e4m3(np.arange(0x80, 0xff, dtype=np.uint8))
    assert np.array_equal(neg, -pos)
    fin = F.decode_e4m3(np.array([c for c in range(256) if c not in (0x7f, 0xff)], np.uint8))
    as_bf16 = torch.from_numpy(fin).float().to(torch.bfloat16).double().numpy()
    assert np.array_equal(as_bf16, fin)


@pytest.mark.parametrize("V", [4096, 32064])
def test_uniform_logits_through_codes(V):
    T, H = 5, 32
    rng = np.random.default_rng(0)
    h = rng.integers(0, 0x7e, size=(T, H)).astype(np.uint8)
    W = np.zeros((V, H), np.uint8)
    lp, ent, lse = F.forward(h, 0.37, W, 1.9, rng.integers(0, V, size=T))
    assert np.allclose(lp, -math.log(V), atol=1e-12, rtol=0)
    assert np.allclose(ent, math.log(V), atol=1e-12, rtol=0)


def check_dominant(forward):
    V, H, k = 4096, 16, 77
    h = np.zeros((1, H), np.uint8)
    h[0, 0] = 0x40                  # 2.0
    W = np.zeros((V, H), np.uint8)
    W[k, 0] = 0x58                  # 16.0
    s_h, s_w = 0.25, 2.0            # d = 0.25 * 2 * 2 * 16 = 16
    d = 16.0
    lp, ent, lse = forward(h, s_h, W, s_w, np.array([k]))
    ref_lse = math.log(math.exp(d) + V - 1)
    assert abs(lse[0] - ref_lse) < 1e-12
    assert abs(lp[0] - (d - ref_lse)) < 1e-12
    assert abs(ent[0] - (ref_lse - d * math.exp(d - ref_lse))) < 1e-12
    # the other tokens' log-prob: -lse
    lp2, _, _ = forward(h, s_h, W, s_w, np.array([k + 1]))
    assert abs(lp2[0] + ref_lse) < 1e-12


def test_dominant_logit_through_codes_and_scales():
    check_dominant(F.forward)


def _decode_bias8(codes):
    """The FNUZ variant's exponent bias (8) in place of E4M3's 7."""
    return F.decode_e4m3(codes) / 2.0


def _decode_nan_at_negative_zero(codes):
    v = F.decode_e4m3(codes)
    return np.where(np.asarray(codes, np.uint8) == 0x80, np.nan, v)


def _forward_scale_h_twice(h, s_h, W, s_w, y):
    return F.lmhead.forward(F.dequantize(h, s_h), F.dequantize(W, s_h), y)


def _forward_scales_dropped(h, s_h, W, s_w, y):
    return F.lmhead.forward(F.decode_e4m3(h), F.decode_e4m3(W), y)


@pytest.mark.parametrize("bad", [_decode_bias8, _decode_nan_at_negative_zero])
def test_planted_decode_mistakes_fail_the_code_pin(bad):
    with pytest.raises(AssertionError):
        check_codes(bad)


@pytest.mark.parametrize("bad", [_forward_scale_h_twice, _forward_scales_dropped])
def test_planted_scale_mistakes_fail_the_closed_form(bad):
    with pytest.raises(AssertionError):
        check_dominant(bad)


def test_backward_is_with_respect_to_the_dequantized_values():
    """Central differences of the loss in the dequantized h and W (the codes are not
    differentiable; the gradient is taken in the values they stand for)."""
    from oracle import lmhead as O
    rng = np.random.default_rng(3)
    T, H, V = 4, 6, 9
    hc = rng.integers(0, 0x60, size=(T, H)).astype(np.uint8) | (rng.integers(0, 2, size=(T, H)) << 7).astype(np.uint8)
    Wc = rng.integers(0, 0x50, size=(V, H)).astype(np.uint8)
    s_h, s_w = 0.05, 0.01
    y = rng.integers(0, V, size=T)
    m = np.array([1, 0, 1, 1], np.uint8)
    a, b = rng.uniform(-1, 1, T), rng.uniform(-1, 1, T)
    dH, dW = F.backward(hc, s_h, Wc, s_w, y, m, a, b)
    h, W = F.dequantize(hc, s_h), F.dequantize(Wc, s_w)
    eps = 1e-6
    for (t, j) in [(0, 0), (2, 5), (3, 3)]:
        hp, hm = h.copy(), h.copy()
        hp[t, j] += eps
        hm[t, j] -= eps
        fd = (O.loss(hp, W, y, m, a, b) - O.loss(hm, W, y, m, a, b)) / (2 * eps)
        assert abs(fd - dH[t, j]) <= 1e-6 * max(1.0, abs(fd))
    for (v, j) in [(0, 1), (8, 4)]:
        Wp, Wm = W.copy(), W.copy()
        Wp[v, j] += eps
        Wm[v, j] -= eps
        fd = (O.loss(h, Wp, y, m, a, b) - O.loss(h, Wm, y, m, a, b)) / (2 * eps)
        assert abs(fd - dW[v, j]) <= 1e-6 * max(1.0, abs(fd))
    assert not dH[1].any()


def test_input_generator_codes_decode_near_the_fp32_draws():
    from workloads import make_tensors, make_tensors_fp8
    hc, s_h, Wc, s_w, y = make_tensors_fp8(64, 32, 300, 5)
    h, W, y2 = make_tensors(64, 32, 300, "f32", 5)
    assert torch.equal(y, y2) and hc.dtype == torch.uint8
    hv = F.dequantize(hc.numpy(), s_h)
    # E4M3 keeps 3 mantissa bits: relative rounding error <= 2^-4 above the subnormals
    err = np.abs(hv - h.double().numpy())
    assert np.all(err <= 2.0 ** -4 * np.abs(h.double().numpy()) + s_h * 2.0 ** -9)
    assert np.isfinite(hv).all() and np.abs(F.decode_e4m3(Wc.numpy())).max() <= 448.0
