"""Seeded hidden states, weights, targets and upstream gradients.

h ~ N(0, 1) and W ~ N(0, 0.02^2) are drawn in float32 and, for bf16 workloads,
rounded to bfloat16 (round to nearest even); targets ~ U{0..V-1}.  Draws use a
``torch.Generator`` on the requested device, so large inputs are made where they
are used.  The oracle then reads back exactly the stored bytes.
"""

from __future__ import annotations

from typing import Optional, Tuple

import numpy as np
import torch

_DT = {"f32": torch.float32, "bf16": torch.bfloat16}


def make_tensors(T: int, H: int, V: int, dtype: str, seed: int,
                 device="cpu") -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """Returns (h [T,H], W [V,H], targets int64 [T]) on ``device``."""
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    h = torch.randn((T, H), generator=g, device=device, dtype=torch.float32)
    W = torch.randn((V, H), generator=g, device=device, dtype=torch.float32).mul_(0.02)
    y = torch.randint(0, V, (T,), generator=g, device=device, dtype=torch.int64)
    dt = _DT[dtype]
    if dt != torch.float32:
        h = h.to(dt)
        W = W.to(dt)
    return h.contiguous(), W.contiguous(), y


def make_upstream(mask: np.ndarray, mode: str = "lp+ent",
                  seed: Optional[int] = None) -> Tuple[np.ndarray, Optional[np.ndarray]]:
    """Upstream gradients of (logprob, entropy), float32 [T].

    "lp+ent": a = b = 1/A on active tokens, 0 elsewhere (A = active count).
    "lp":     a as above, no entropy gradient (None).
    "random": a, b ~ U(-1, 1) on every token (the loss mask still gates them).
    """
    m = (np.asarray(mask) != 0)
    T = m.shape[0]
    if mode == "random":
        rng = np.random.default_rng(0 if seed is None else seed)
        a = rng.uniform(-1.0, 1.0, T).astype(np.float32)
        b = rng.uniform(-1.0, 1.0, T).astype(np.float32)
        return a, b
    A = int(m.sum())
    a = np.zeros(T, np.float32)
    if A:
        a[m] = np.float32(1.0 / A)
    if mode == "lp":
        return a, None
    if mode != "lp+ent":
        raise ValueError(mode)
    return a, a.copy()


def make_tensors_fp8(T: int, H: int, V: int, seed: int, device="cpu"):
    """FP8 inputs: (h codes uint8 [T,H], scale_h, W codes uint8 [V,H], scale_w,
    targets int64 [T]).

    h and W are drawn exactly as by make_tensors (same seed, fp32), then each tensor
    is given one fp32 scale, amax / 448 (448 = the largest finite OCP E4M3 value), and
    rounded to E4M3 codes of x / scale by torch's float8_e4m3fn conversion."""
    h, W, y = make_tensors(T, H, V, "f32", seed, device=device)
    out = []
    for x in (h, W):
        scale = float(x.abs().max().clamp_min(1e-30)) / 448.0
        scale = float(np.float32(scale))
        codes = (x / scale).to(torch.float8_e4m3fn).view(torch.uint8).contiguous()
        out += [codes, scale]
    return out[0], out[1], out[2], out[3], y
