"""Seeded loss masks shaped like packed RL/SFT batches.

Every mask is a flat ``uint8[T]`` row (1 = token contributes to the loss).
Packed sequence lengths are drawn i.i.d. until T is filled; the last sequence
is truncated; no alignment padding.  Each recipe is retried with seed+k
(k = 0, 1, ...) until its active fraction falls inside the config's band; the
k used is returned in the info dict.
"""

from __future__ import annotations

from typing import Dict, List, Optional, Tuple

import numpy as np

from .configs import get_config


def _lengths(rng: np.random.Generator, T: int, lo: int, hi: int) -> List[int]:
    out, n = [], 0
    while n < T:
        L = min(int(rng.integers(lo, hi + 1)), T - n)
        out.append(L)
        n += L
    return out


def _punch_gaps(m: np.ndarray, rng: np.random.Generator, lo: int, hi_excl: int,
                rate: float, gmax: int) -> None:
    """Clear random gaps of U{1..gmax} tokens inside m[lo:hi_excl] (a response)."""
    R = hi_excl - lo
    if R <= 0:
        return
    for _ in range(int(rng.poisson(rate * R))):
        s = lo + int(rng.integers(0, R))
        g = int(rng.integers(1, gmax + 1))
        m[s:min(hi_excl, s + g)] = 0


def _tiny(rng, T):
    m = np.zeros(T, np.uint8)
    for s in range(0, T, 128):
        m[s + 48:s + 128] = 1
    return m, {"n_seqs": T // 128}


def _llama(rng, T):
    m = np.zeros(T, np.uint8)
    pos = 0
    L_all = _lengths(rng, T, 512, 4096)
    for L in L_all:
        P = int(round(rng.uniform(0.2, 0.6) * L))
        m[pos + P:pos + L] = 1
        _punch_gaps(m, rng, pos + P, pos + L, 0.0022, 300)
        pos += L
    return m, {"n_seqs": len(L_all)}


def _tp4_share(rng, T):
    m = np.zeros(T, np.uint8)
    pos = 0
    L_all = _lengths(rng, T, 1024, 8192)
    for L in L_all:
        if rng.random() < 0.5:          # short-tail response
            R = min(L, int(rng.integers(16, 257)))
            m[pos + L - R:pos + L] = 1
        else:
            P = int(round(rng.uniform(0.2, 0.6) * L))
            m[pos + P:pos + L] = 1
        pos += L
    return m, {"n_seqs": len(L_all)}


def _wide_vocab(rng, T):
    m = np.zeros(T, np.uint8)
    pos = 0
    L_all = _lengths(rng, T, 4096, 16384)
    for L in L_all:
        P = int(round(rng.uniform(0.2, 0.5) * L))
        m[pos + P:pos + L] = 1
        _punch_gaps(m, rng, pos + P, pos + L, 0.001, 128)
        pos += L
    return m, {"n_seqs": len(L_all)}


def _stress(rng, T, frac):
    """Alternating renewal on the flat row: active runs ~ Geometric(mean 200),
    gaps ~ Geometric(mean 150) (base active share 4/7).  For frac <= 4/7 each
    run is kept with probability frac / (4/7); above, each gap is filled with
    probability (350 frac - 200) / 150; frac == 1 is all-active."""
    if frac >= 1.0:
        return np.ones(T, np.uint8), {"runs": 1}
    m = np.zeros(T, np.uint8)
    base = 200.0 / 350.0
    keep = min(1.0, frac / base)
    fill = max(0.0, (350.0 * frac - 200.0) / 150.0)
    pos, runs = 0, 0
    active = bool(rng.random() < base)
    while pos < T:
        if active:
            n = int(rng.geometric(1.0 / 200.0))
            if rng.random() < keep:
                m[pos:pos + n] = 1
                runs += 1
        else:
            n = int(rng.geometric(1.0 / 150.0))
            if fill > 0.0 and rng.random() < fill:
                m[pos:pos + n] = 1
        pos += n
        active = not active
    return m, {"runs": runs}


_BANDS = {0.05: 0.015, 0.25: 0.03, 0.50: 0.03, 0.90: 0.03, 1.00: 0.0}


def make_mask(cid: int, active_frac: Optional[float] = None, T: Optional[int] = None,
              seed: Optional[int] = None, max_tries: int = 64) -> Tuple[np.ndarray, Dict]:
    """Loss mask for config ``cid`` (1..5).  ``active_frac`` selects a point of
    the stress sweep (config 5 only).  ``T`` overrides the length (same recipe,
    no calibration band) for reduced-size tests."""
    cfg = get_config(cid)
    T_use = cfg.T if T is None else int(T)
    base_seed = cfg.seed if seed is None else int(seed)
    if cid == 5:
        frac = cfg.target_active if active_frac is None else float(active_frac)
        target, band = frac, _BANDS.get(round(frac, 2), 0.03)
    else:
        if active_frac is not None:
            raise ValueError("active_frac applies to the stress workload only")
        target, band = cfg.target_active, cfg.band
    calibrate = T is None and band > 0.0
    for k in range(max_tries):
        rng = np.random.default_rng(base_seed + k)
        if cid == 1:
            m, info = _tiny(rng, T_use)
        elif cid == 2:
            m, info = _llama(rng, T_use)
        elif cid == 3:
            m, info = _tp4_share(rng, T_use)
        elif cid == 4:
            m, info = _wide_vocab(rng, T_use)
        else:
            m, info = _stress(rng, T_use, target)
        frac_got = float(m.mean()) if T_use else 0.0
        if not calibrate or abs(frac_got - target) <= band:
            info.update({"seed": base_seed + k, "retry": k, "active_frac": frac_got,
                         "target_active": target})
            return m, info
    raise RuntimeError(f"mask recipe for config {cid} missed its band after {max_tries} tries")
