"""FP8 (OCP E4M3) inputs: the value of each code, and the fused LM head on the values.

TEST INFRASTRUCTURE ONLY -- see the package docstring.

The pages list FP8 among the layouts the span builder serves (SkyRL #2376, Bugbot
"Overview": packed TP/CP/FP8 layouts) but give no recipe for FP8 inputs.  Reading
taken here: h and W arrive as 8-bit codes of the OCP E4M3 format (the variant
without infinities) with one fp32 scale per tensor,

    h[t, k] = scale_h * value(h_code[t, k]),   W[v, k] = scale_w * value(W_code[v, k]),

and the method computes on those values exactly what it computes for any other
input dtype, so the oracle is the plain definition of :mod:`oracle.lmhead` applied
to the decoded, scaled values in float64.  Gradients are taken with respect to
those values (the codes themselves are not differentiable).

E4M3 (OCP 8-bit floating point, E4M3): bit 7 is the sign; bits 6..3 the exponent e
with bias 7; bits 2..0 the mantissa m.  e = 0 encodes the subnormals m/8 * 2^-6
(m = 0: zero, signed); e = 1..15 encodes (1 + m/8) * 2^(e - 7), except that e = 15,
m = 7 is NaN.  There is no infinity; the largest finite value is 1.75 * 2^8 = 448.
"""

from __future__ import annotations

from typing import Tuple

import numpy as np

from . import lmhead


def decode_e4m3(codes) -> np.ndarray:
    """uint8 E4M3 codes -> the float64 values they encode (NaN for the NaN codes)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = c >> 7
    e = (c >> 3) & 15
    m = c & 7
    mag = np.where(e == 0, (m / 8.0) * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return np.where(sign == 1, -mag, mag)


def dequantize(codes, scale) -> np.ndarray:
    """scale * value(code), with the scale taken as the fp32 number the caller passes
    (a 24-bit significand times a 4-bit one: exact in float64)."""
    return float(np.float32(scale)) * decode_e4m3(codes)


def forward(h_codes, scale_h, W_codes, scale_w, targets,
            block: int = 64) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """(logprob, entropy, lse) of the fused LM head on the dequantized h and W."""
    return lmhead.forward(dequantize(h_codes, scale_h), dequantize(W_codes, scale_w), targets, block=block)


def backward(h_codes, scale_h, W_codes, scale_w, targets, loss_mask, grad_logprob, grad_entropy,
             block: int = 64) -> Tuple[np.ndarray, np.ndarray]:
    """(dH, dW) with respect to the dequantized h and W."""
    return lmhead.backward(dequantize(h_codes, scale_h), dequantize(W_codes, scale_w), targets, loss_mask,
                           grad_logprob, grad_entropy, block=block)
