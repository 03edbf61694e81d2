"""The HIP path at the full workload sizes, in the launch configuration bench.py times.

At full size the fp64 oracle cannot afford every output, so:

* spans, tile bitmap and active count: bit-exact against the oracle over all T;
* forward outputs (logprob, entropy, lse) and d_hidden rows: on 256 sampled tokens
  (first/last tokens, 128-token tile edges, span starts and ends, and random ones),
  against the oracle's per-token definitions, which are exact at any T because each
  token's outputs depend on its own hidden row alone (SkyRL #2376, "How it works");
* every inactive d_hidden row: bitwise +0;
* the forward over active token tiles only (FLH_FWD_SKIP_INACTIVE): the dense outputs
  bitwise on active tiles, zeros elsewhere;
* the weight gradient over active token tiles only (FLH_BWD_SKIP_INACTIVE_DW): d_hidden
  and d_weight bitwise equal to the dense mode's;
* d_weight, which depends on every token, through identities that hold at any size:
  each row of the d-logits sums to zero over the vocabulary (both the log-prob and the
  entropy terms do), so sum_v dW[v, :] = 0; and <dH, h> = <dW, W> = sum D * z.

The tolerances are the ones of the reduced-size parity tests: max abs 5e-3 for the
forward outputs and relative Frobenius 1e-2 for the gradient rows.

T-slices of configs 2-5 (1024 tokens chosen to straddle active and inactive runs) are
also checked against the full oracle at full H and V, d_weight tile by tile as well.
The long weight-gradient loop (K = T) is checked element by element at the stress
workload's full T with small H and V, where the oracle can afford every output.

Every d_weight entry at full T, H and V: tokens enter the loss independently, so with the
upstream gradients zero outside 256 sampled tokens the full-size d_weight is exactly the
oracle's weight gradient of those 256 tokens alone, which the oracle can afford; the kernels
still run the whole workload (every active tile, K = T), so a lost or misplaced 256 x 256
block of d_weight, or a wrong stage of the long contraction, shows.
"""

import numpy as np
import pytest
import torch

from entropy_block_sparse_amd import flh_backward, flh_forward, flh_spans_build
from oracle import lmhead as O
from oracle import spans as S
from tests.gpu_common import announce, cuda_device, host64
from tests.helpers import max_abs, rel_fro
from workloads import CONFIGS, make_mask, make_tensors, make_upstream

pytestmark = pytest.mark.gpu

TOL_LP = 5e-3
TOL_GRAD = 1e-2
MAX_GAP = 128
TILE_M = 128


def _sample_tokens(mask, n=256, seed=0):
    T = len(mask)
    rng = np.random.default_rng(seed)
    picks = {0, T - 1}
    for t in (TILE_M - 1, TILE_M, 2 * TILE_M - 1, 2 * TILE_M, T - TILE_M - 1, T - TILE_M):
        if 0 <= t < T:
            picks.add(t)
    for s, e in S.active_spans(mask, MAX_GAP)[:24]:
        picks.update({s, e - 1, max(s - 1, 0), min(e, T - 1)})
    act = np.nonzero(mask)[0]
    if len(act):
        picks.update(int(x) for x in rng.choice(act, size=min(len(act), n // 2), replace=False))
    picks.update(int(x) for x in rng.integers(0, T, size=n))
    return np.array(sorted(picks)[:n], dtype=np.int64)


def _slice_window(mask, L):
    """A window of L tokens whose active fraction is closest to one half."""
    T = len(mask)
    c = np.concatenate([[0], np.cumsum(mask, dtype=np.int64)])
    starts = np.arange(0, T - L + 1, 64)
    frac = (c[starts + L] - c[starts]) / L
    return int(starts[np.argmin(np.abs(frac - 0.5))])


def tile_rel_fro(got, ref, tile=256):
    """Largest relative Frobenius error over the tile x tile blocks of a matrix whose
    reference block is not zero: a block the kernel lost or misplaced scores ~1."""
    worst = 0.0
    for r in range(0, ref.shape[0], tile):
        for c in range(0, ref.shape[1], tile):
            o = ref[r:r + tile, c:c + tile]
            den = np.linalg.norm(o)
            if den > 0:
                worst = max(worst, float(np.linalg.norm(got[r:r + tile, c:c + tile] - o) / den))
    return worst


TOL_TILE = 2e-2

FULL = [(2, None, False), (3, None, False), (4, None, False), (5, 0.05, False), (5, 0.5, False),
        (5, 0.9, False), (5, 1.0, False), (5, 1.0, True)]


@pytest.mark.parametrize("cid,frac,dense", FULL)
def test_full_size_spot_checks(cid, frac, dense):
    """dense: the fallback without metadata (meta=NULL), which at 100% active must give
    the span path's results bitwise."""
    cfg = CONFIGS[cid]
    dev = cuda_device()
    mask, _ = make_mask(cid, active_frac=frac)
    T, H, V = cfg.T, cfg.H, cfg.V
    announce(f"full size config {cid} T={T} H={H} V={V} split={cfg.vocab_split} active={mask.mean():.3f} "
             f"dense_fallback={dense}")
    h, W, y = make_tensors(T, H, V, cfg.dtype, cfg.seed, device=dev)
    a, b = make_upstream(mask)
    m_dev = torch.as_tensor(mask).to(dev)
    meta = flh_spans_build(m_dev)
    lp, ent, lse = flh_forward(h, W, y)
    dH, dW = flh_backward(h, W, y, lse, ent, torch.as_tensor(a).to(dev), torch.as_tensor(b).to(dev),
                          m_dev, None if dense else meta, cfg.vocab_split)
    torch.cuda.synchronize()
    if dense:
        # the dense fallback computes every token tile and one span over all tokens: at
        # 100% active that is the span path's work in the same order
        assert mask.all()
        dHs, dWs = flh_backward(h, W, y, lse, ent, torch.as_tensor(a).to(dev), torch.as_tensor(b).to(dev),
                                m_dev, meta, cfg.vocab_split)
        torch.cuda.synchronize()
        assert torch.equal(dH, dHs) and torch.equal(dW, dWs)
        del dHs, dWs

    # active metadata: bit-exact
    assert meta.host_spans() == S.active_spans(mask, MAX_GAP)
    assert int(meta.active_count.item()) == int(mask.sum())
    bits = meta.tile_bits.cpu().numpy().view(np.uint32)
    ref_bits = S.tile_bits(mask, TILE_M)
    assert np.array_equal(bits[:len(ref_bits)], ref_bits)

    # forward and d_hidden rows on sampled tokens
    rows = _sample_tokens(mask, seed=cid)
    Wf = host64(W)
    hr = host64(h[torch.as_tensor(rows, device=dev)])
    yr = y.cpu().numpy()[rows]
    olp, oent, olse = O.forward(hr, Wf, yr)
    assert max_abs(lp.cpu().numpy()[rows], olp) <= TOL_LP
    assert max_abs(ent.cpu().numpy()[rows], oent) <= TOL_LP
    assert max_abs(lse.cpu().numpy()[rows], olse) <= TOL_LP
    act = rows[mask[rows] != 0]
    if len(act):
        sel = np.searchsorted(rows, act)
        odH = O.dhidden_rows(hr[sel], Wf, yr[sel], mask[act], a[act], b[act], range(len(act)))
        gdH = host64(dH[torch.as_tensor(act, device=dev)])
        assert rel_fro(gdH, odH) <= TOL_GRAD, rel_fro(gdH, odH)
    del Wf

    # every inactive d_hidden row is bitwise +0
    inactive = torch.as_tensor(mask == 0, device=dev)
    raw = dH.view(torch.int16)
    assert not bool((raw[inactive] != 0).any()), "inactive d_hidden rows must be bitwise +0"

    # d_weight identities, evaluated in fp64 on the device from the stored outputs
    dW64 = dW.double()
    col_sum = dW64.sum(dim=0)
    col_abs = dW64.abs().sum(dim=0)
    assert float((col_sum.abs() / col_abs.clamp_min(1e-300)).max()) <= 1e-2
    lhs = float((dH.double() * h.double()).sum())
    rhs = float((dW64 * W.double()).sum())
    assert abs(lhs - rhs) <= 1e-2 * max(abs(lhs), abs(rhs)), (lhs, rhs)
    del dW64

    # the forward over active token tiles only: the dense outputs on those tiles, 0 elsewhere
    sp = flh_forward(h, W, y, meta=meta, skip_inactive=True)
    torch.cuda.synchronize()
    tiles = np.zeros(-(-T // 128), bool)
    tiles[np.nonzero(mask)[0] // 128] = True
    act_dev = torch.as_tensor(np.repeat(tiles, 128)[:T]).to(dev)
    for d, s in zip((lp, ent, lse), sp):
        assert torch.equal(d[act_dev], s[act_dev]) and not s[~act_dev].any()
    del sp

    # the weight gradient over active token tiles only equals the dense one bitwise
    dH2, dW2 = flh_backward(h, W, y, lse, ent, torch.as_tensor(a).to(dev), torch.as_tensor(b).to(dev),
                            m_dev, meta, cfg.vocab_split, skip_inactive_dw=True)
    torch.cuda.synchronize()
    assert torch.equal(dH, dH2) and torch.equal(dW, dW2)
    del dH, dW, dH2, dW2, h, W
    torch.cuda.empty_cache()


@pytest.mark.parametrize("cid,frac", [(2, None), (3, None), (4, None), (5, 0.25)])
def test_full_hv_t_slice_against_oracle(cid, frac):
    cfg = CONFIGS[cid]
    dev = cuda_device()
    L = 1024
    mask_full, _ = make_mask(cid, active_frac=frac)
    t0 = _slice_window(mask_full, L)
    mask = np.ascontiguousarray(mask_full[t0:t0 + L])
    announce(f"T-slice config {cid} tokens [{t0}, {t0 + L}) H={cfg.H} V={cfg.V} active={mask.mean():.3f}")
    h_full, W, y_full = make_tensors(cfg.T, cfg.H, cfg.V, cfg.dtype, cfg.seed, device=dev)
    h = h_full[t0:t0 + L].contiguous()
    y = y_full[t0:t0 + L].contiguous()
    del h_full, y_full
    a, b = make_upstream(mask)
    m_dev = torch.as_tensor(mask).to(dev)
    meta = flh_spans_build(m_dev)
    lp, ent, lse = flh_forward(h, W, y)
    dH, dW = flh_backward(h, W, y, lse, ent, torch.as_tensor(a).to(dev), torch.as_tensor(b).to(dev),
                          m_dev, meta, cfg.vocab_split)
    torch.cuda.synchronize()
    hh, WW, yy = host64(h), host64(W), y.cpu().numpy()
    olp, oent, olse = O.forward(hh, WW, yy)
    assert max_abs(lp.cpu().numpy(), olp) <= TOL_LP
    assert max_abs(ent.cpu().numpy(), oent) <= TOL_LP
    assert max_abs(lse.cpu().numpy(), olse) <= TOL_LP
    odH, odW = O.backward(hh, WW, yy, mask, a, b)
    gdW = host64(dW)
    assert rel_fro(host64(dH), odH) <= TOL_GRAD
    assert rel_fro(gdW, odW) <= TOL_GRAD
    # every 256 x 256 block of d_weight on its own: a lost or misplaced block fails here
    assert tile_rel_fro(gdW, odW) <= TOL_TILE, tile_rel_fro(gdW, odW)
    raw = dH.view(torch.int16).cpu().numpy()
    assert not raw[mask == 0].any()
    del dH, dW, W, h
    torch.cuda.empty_cache()


@pytest.mark.parametrize("frac", [0.05, 0.9])
def test_long_token_axis_against_full_oracle(frac):
    """The stress workload's full T = 262144 and its mask, at H = 64 and V = 2048 where
    the fp64 oracle computes every output: the weight gradient's contraction runs over
    all 262144 tokens (4096 K stages), checked entry by entry, as are every d_hidden row
    and every forward output.  Four vocabulary splits of 512."""
    dev = cuda_device()
    mask, _ = make_mask(5, active_frac=frac)
    T, H, V, split = len(mask), 64, 2048, 512
    announce(f"long token axis T={T} H={H} V={V} split={split} active={mask.mean():.3f}")
    h, W, y = make_tensors(T, H, V, "bf16", 4242, device=dev)
    a, b = make_upstream(mask)
    m_dev = torch.as_tensor(mask).to(dev)
    meta = flh_spans_build(m_dev)
    lp, ent, lse = flh_forward(h, W, y)
    dH, dW = flh_backward(h, W, y, lse, ent, torch.as_tensor(a).to(dev), torch.as_tensor(b).to(dev),
                          m_dev, meta, split)
    torch.cuda.synchronize()
    hh, WW, yy = host64(h), host64(W), y.cpu().numpy()
    olp, oent, olse = O.forward(hh, WW, yy, block=1024)
    assert max_abs(lp.cpu().numpy(), olp) <= TOL_LP
    assert max_abs(ent.cpu().numpy(), oent) <= TOL_LP
    assert max_abs(lse.cpu().numpy(), olse) <= TOL_LP
    odH, odW = O.backward(hh, WW, yy, mask, a, b, block=1024)
    gdH, gdW = host64(dH), host64(dW)
    assert rel_fro(gdW, odW) <= TOL_GRAD
    assert tile_rel_fro(gdW, odW) <= TOL_TILE
    # entry by entry: bf16 rounding of the d-logits and of d_weight, fp32 sums over
    # 262144 tokens; the floor (1% of the rms entry) covers entries that nearly cancel
    rms = float(np.sqrt((odW ** 2).mean()))
    err = np.abs(gdW - odW)
    bad = err > 2e-2 * np.abs(odW) + 1e-2 * rms
    assert not bad.any(), (int(bad.sum()), float(err.max()), rms)
    assert rel_fro(gdH, odH) <= TOL_GRAD
    act = np.nonzero(mask)[0]
    num = np.linalg.norm(gdH[act] - odH[act], axis=1)
    den = np.linalg.norm(odH[act], axis=1)
    assert np.all(num <= 3e-2 * den + 1e-12)
    assert not dH.view(torch.int16).cpu().numpy()[mask == 0].any()


def _sampled_upstream(mask, n, seed):
    """Upstream gradients zero except on n sampled tokens (n - 16 active, 16 inactive, which
    the mask must silence), the samples spread over all of T."""
    rng = np.random.default_rng(seed)
    act = np.nonzero(mask)[0]
    ina = np.nonzero(mask == 0)[0]
    pick = set(int(x) for x in rng.choice(act, size=min(len(act), n - 16), replace=False))
    pick.update((int(act[0]), int(act[-1])))
    if len(ina):
        pick.update(int(x) for x in rng.choice(ina, size=min(len(ina), 16), replace=False))
    rows = np.array(sorted(pick), dtype=np.int64)
    a_full, b_full = make_upstream(mask)
    a = np.zeros_like(a_full)
    b = np.zeros_like(b_full)
    a[rows] = a_full[rows]
    b[rows] = b_full[rows]
    off = rows[mask[rows] == 0]
    a[off], b[off] = 0.75, -0.5  # nonzero upstream on inactive tokens: the mask must zero it
    return rows, a, b


@pytest.mark.parametrize("cid,frac", [(2, None), (4, None), (5, 0.5)])
def test_full_size_dweight_every_entry_on_sampled_upstream(cid, frac):
    """Full-size d_weight entry by entry (and tile by tile) against the oracle's backward of
    256 sampled tokens, the upstream gradients being zero elsewhere; d_hidden: the sampled
    active rows against the oracle, every other row exactly zero."""
    cfg = CONFIGS[cid]
    dev = cuda_device()
    mask, _ = make_mask(cid, active_frac=frac)
    T, H, V = cfg.T, cfg.H, cfg.V
    announce(f"full-size dW, sampled upstream: config {cid} T={T} H={H} V={V} split={cfg.vocab_split}")
    h, W, y = make_tensors(T, H, V, cfg.dtype, cfg.seed, device=dev)
    rows, a, b = _sampled_upstream(mask, 256, seed=100 + cid)
    m_dev = torch.as_tensor(mask).to(dev)
    meta = flh_spans_build(m_dev)
    lp, ent, lse = flh_forward(h, W, y)
    dH, dW = flh_backward(h, W, y, lse, ent, torch.as_tensor(a).to(dev), torch.as_tensor(b).to(dev),
                          m_dev, meta, cfg.vocab_split)
    torch.cuda.synchronize()
    # d_hidden: zero outside the sampled active rows (value zero: an active row with zero
    # upstream sums products 0 * x)
    keep = np.zeros(T, bool)
    keep[rows[mask[rows] != 0]] = True
    assert not bool((dH[torch.as_tensor(~keep, device=dev)] != 0).any())
    hr = host64(h[torch.as_tensor(rows, device=dev)])
    yr = y.cpu().numpy()[rows]
    gdH = host64(dH[torch.as_tensor(rows, device=dev)])
    del dH, h
    Wf = host64(W)
    del W
    odH, odW = O.backward(hr, Wf, yr, mask[rows], a[rows], b[rows])
    del Wf
    act = mask[rows] != 0
    assert rel_fro(gdH[act], odH[act]) <= TOL_GRAD
    assert not gdH[~act].any() and not odH[~act].any()
    gdW = host64(dW)
    del dW
    torch.cuda.empty_cache()
    assert rel_fro(gdW, odW) <= TOL_GRAD, rel_fro(gdW, odW)
    worst = tile_rel_fro(gdW, odW)
    assert worst <= TOL_TILE, worst


def _renewal_mask(T, seed, mean_run=175):
    """Alternating active / inactive runs of geometric length (mean `mean_run`), vectorised."""
    rng = np.random.default_rng(seed)
    lens = rng.geometric(1.0 / mean_run, size=2 * (T // mean_run) + 64)
    ends = np.cumsum(lens)
    lens = lens[:int(np.searchsorted(ends, T)) + 1]
    starts = np.concatenate([[0], np.cumsum(lens)[:-1]])
    m = np.zeros(T, np.uint8)
    for s, n in zip(starts[1::2], lens[1::2]):  # odd runs active, the first run inactive
        m[s:min(T, s + n)] = 1
    return m


def test_largest_token_count():
    """T = 2^24 - 128, the largest token count the library accepts (below 2^24), with small H
    and V: the backward's transposed operands then have rows of about 2^24 elements, so a
    wave's 64 rows reach byte offsets near 2^31.  Spans and tile bits bit-exact over all T;
    upstream gradients zero outside 258 sampled tokens, so every d_weight entry is the
    oracle's gradient of those tokens alone; forward outputs and d_hidden rows on the
    sampled tokens, every other d_hidden row exactly zero."""
    T, H, V, split = (1 << 24) - 128, 64, 2048, 512
    dev = cuda_device()
    announce(f"largest T: T={T} H={H} V={V} split={split}")
    mask = _renewal_mask(T, seed=2024)
    h, W, y = make_tensors(T, H, V, "bf16", 2025, device=dev)
    rows, a, b = _sampled_upstream(mask, 256, seed=2026)
    m_dev = torch.as_tensor(mask).to(dev)
    meta = flh_spans_build(m_dev)
    lp, ent, lse = flh_forward(h, W, y)
    dH, dW = flh_backward(h, W, y, lse, ent, torch.as_tensor(a).to(dev), torch.as_tensor(b).to(dev),
                          m_dev, meta, split)
    torch.cuda.synchronize()
    assert meta.host_spans() == S.active_spans(mask, MAX_GAP)
    assert int(meta.active_count.item()) == int(mask.sum())
    ref_bits = S.tile_bits(mask, TILE_M)
    assert np.array_equal(meta.tile_bits.cpu().numpy().view(np.uint32)[:len(ref_bits)], ref_bits)
    keep = np.zeros(T, bool)
    keep[rows[mask[rows] != 0]] = True
    assert not bool((dH[torch.as_tensor(~keep, device=dev)] != 0).any())
    ridx = torch.as_tensor(rows, device=dev)
    hr, yr = host64(h[ridx]), y.cpu().numpy()[rows]
    Wf = host64(W)
    olp, oent, olse = O.forward(hr, Wf, yr)
    assert max_abs(lp.cpu().numpy()[rows], olp) <= TOL_LP
    assert max_abs(ent.cpu().numpy()[rows], oent) <= TOL_LP
    assert max_abs(lse.cpu().numpy()[rows], olse) <= TOL_LP
    odH, odW = O.backward(hr, Wf, yr, mask[rows], a[rows], b[rows])
    act = mask[rows] != 0
    assert rel_fro(host64(dH[ridx])[act], odH[act]) <= TOL_GRAD
    gdW = host64(dW)
    assert rel_fro(gdW, odW) <= TOL_GRAD
    assert tile_rel_fro(gdW, odW) <= TOL_TILE
    del h, W, dH, dW
    torch.cuda.empty_cache()
