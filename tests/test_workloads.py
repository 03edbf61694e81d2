"""Synthetic workload generator checks (CPU only): seeded, deterministic, and
shaped as the mask recipes state (active-fraction bands, span structure)."""

import numpy as np
import pytest
import torch

from oracle import spans as S
from workloads import CONFIGS, make_mask, make_tensors, make_upstream


def test_tiny_mask_exact():
    m, info = make_mask(1)
    want = np.zeros(512, np.uint8)
    for s in range(0, 512, 128):
        want[s + 48:s + 128] = 1
    assert np.array_equal(m, want) and info["active_frac"] == 0.625


@pytest.mark.parametrize("cid", [2, 3, 4])
def test_mask_bands_and_determinism(cid):
    cfg = CONFIGS[cid]
    m, info = make_mask(cid)
    assert m.shape == (cfg.T,) and m.dtype == np.uint8
    assert abs(m.mean() - cfg.target_active) <= cfg.band
    m2, _ = make_mask(cid)
    assert np.array_equal(m, m2)


@pytest.mark.parametrize("frac", [0.05, 0.25, 0.5, 0.9, 1.0])
def test_stress_sweep(frac):
    m, info = make_mask(5, active_frac=frac)
    assert m.shape == (262144,)
    band = 0.015 if frac == 0.05 else (0.0 if frac == 1.0 else 0.03)
    assert abs(m.mean() - frac) <= band
    if frac == 1.0:
        assert S.active_spans(m, 128) == [(0, 262144)]


def test_wide_vocab_spans_coalesce_within_responses():
    m, _ = make_mask(4)
    sp = S.active_spans(m, 128)
    runs = S.active_runs(m)
    assert len(sp) < len(runs)          # response gaps <= 128 merge
    assert len(sp) <= 40


def test_reduced_T_override():
    m, info = make_mask(2, T=3000)
    assert m.shape == (3000,) and info["retry"] == 0


def test_tensors_seeded():
    h, W, y = make_tensors(16, 8, 50, "bf16", 99)
    h2, W2, y2 = make_tensors(16, 8, 50, "bf16", 99)
    assert h.dtype == torch.bfloat16 and W.dtype == torch.bfloat16 and y.dtype == torch.int64
    assert torch.equal(h, h2) and torch.equal(W, W2) and torch.equal(y, y2)
    assert int(y.min()) >= 0 and int(y.max()) < 50
    hf, Wf, _ = make_tensors(2000, 64, 3000, "f32", 1)
    assert abs(float(hf.std()) - 1.0) < 0.02 and abs(float(Wf.std()) - 0.02) < 0.0005


def test_upstream_modes():
    m = np.array([0, 1, 1, 0, 1], np.uint8)
    a, b = make_upstream(m)
    assert np.allclose(a, [0, 1 / 3, 1 / 3, 0, 1 / 3]) and np.array_equal(a, b)
    a, b = make_upstream(m, "lp")
    assert b is None
    a, b = make_upstream(np.zeros(4, np.uint8))
    assert not a.any()
