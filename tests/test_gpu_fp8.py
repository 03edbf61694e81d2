"""The FP8 (OCP E4M3) input path against the oracle, through the C ABI.

Inputs are E4M3 codes of h and W with one fp32 scale each (the reading of the pages'
FP8 layouts this library takes, SkyRL #2376 Bugbot "Overview"); the oracle computes on
the decoded, scaled values in float64 (oracle.fp8).  The tolerances are the bf16
path's: logprob, entropy, lse max abs <= 5e-3; d_hidden and d_weight relative Frobenius
<= 1e-2, every active d_hidden row within 3e-2, every 256 x 256 block of d_weight within
2e-2; inactive d_hidden rows bitwise +0.  The fp8 products are exact in fp32, and the
d-logits staging and outputs are bf16 as on the bf16 path, so the same bounds apply.
"""

import numpy as np
import pytest
import torch

from entropy_block_sparse_amd import flh_backward_fp8, flh_forward_fp8, flh_spans_build
from oracle import fp8 as F
from tests.gpu_common import announce, cuda_device, host64
from tests.helpers import max_abs, rel_fro
from workloads import CONFIGS, make_mask, make_tensors_fp8, make_upstream

pytestmark = pytest.mark.gpu

TOL_LP = 5e-3
TOL_GRAD = 1e-2
TOL_TILE = 2e-2


def tile_rel_fro(got, ref, tile=256):
    worst = 0.0
    for r in range(0, ref.shape[0], tile):
        for c in range(0, ref.shape[1], tile):
            o = ref[r:r + tile, c:c + tile]
            den = np.linalg.norm(o)
            if den > 0:
                worst = max(worst, float(np.linalg.norm(got[r:r + tile, c:c + tile] - o) / den))
    return worst


def bursty_mask(T, seed, p_on=0.5, max_run=400):
    rng = np.random.default_rng(seed)
    m = np.zeros(T, np.uint8)
    t, on = 0, bool(rng.random() < p_on)
    while t < T:
        n = int(rng.integers(1, max_run))
        if on:
            m[t:t + n] = 1
        t += n
        on = bool(rng.random() < p_on)
    return m


def run_fp8(T, H, V, mask, split=0, seed=0, mode="lp+ent", use_meta=True, skip_dw=False, check_rows=True):
    dev = cuda_device()
    announce(f"fp8 T={T} H={H} V={V} split={split} mode={mode} meta={use_meta} skip_dw={skip_dw}")
    hc, s_h, Wc, s_w, y = make_tensors_fp8(T, H, V, seed)
    a, b = make_upstream(mask, mode, seed=seed)
    h_d, W_d, y_d = hc.to(dev), Wc.to(dev), y.to(dev)
    m_dev = torch.as_tensor(mask).to(dev)
    lp, ent, lse = flh_forward_fp8(h_d, s_h, W_d, s_w, y_d)
    meta = flh_spans_build(m_dev) if use_meta else None
    dH, dW = flh_backward_fp8(h_d, s_h, W_d, s_w, y_d, lse, ent, torch.as_tensor(a).to(dev),
                              None if b is None else torch.as_tensor(b).to(dev), m_dev, meta, split,
                              skip_inactive_dw=skip_dw)
    torch.cuda.synchronize()
    hn, Wn, yn = hc.numpy(), Wc.numpy(), y.numpy()
    olp, oent, olse = F.forward(hn, s_h, Wn, s_w, yn)
    assert max_abs(lp.cpu().numpy(), olp) <= TOL_LP
    assert max_abs(ent.cpu().numpy(), oent) <= TOL_LP
    assert max_abs(lse.cpu().numpy(), olse) <= TOL_LP
    odH, odW = F.backward(hn, s_h, Wn, s_w, yn, mask, a, b)
    gdH, gdW = host64(dH), host64(dW)
    assert dH.dtype == torch.bfloat16 and dW.dtype == torch.bfloat16
    assert rel_fro(gdH, odH) <= TOL_GRAD, rel_fro(gdH, odH)
    assert rel_fro(gdW, odW) <= TOL_GRAD, rel_fro(gdW, odW)
    if mode != "random":
        assert tile_rel_fro(gdW, odW) <= TOL_TILE, tile_rel_fro(gdW, odW)
    inactive = mask == 0
    if inactive.any():
        assert not dH.view(torch.int16).cpu().numpy()[inactive].any()
    if check_rows and (~inactive).any() and mode != "random":
        act = np.nonzero(~inactive)[0]
        num = np.linalg.norm(gdH[act] - odH[act], axis=1)
        den = np.linalg.norm(odH[act], axis=1)
        assert np.all(num <= 3e-2 * den + 1e-12)
    return dict(lp=lp, ent=ent, lse=lse, dH=dH, dW=dW, meta=meta, h=h_d, W=W_d, y=y_d, s_h=s_h, s_w=s_w)


def test_fp8_ragged_multi_split():
    # T ragged (partial last token tile), H = 528: four K stages of 128 codes and a partial
    # one of 16; three vocabulary splits with a live-width tail of 904
    T, H, V = 1000, 528, 5000
    run_fp8(T, H, V, bursty_mask(T, 3), split=2048, seed=11)


@pytest.mark.parametrize("mode", ["lp", "random"])
def test_fp8_upstream_modes(mode):
    T, H, V = 700, 256, 3000
    run_fp8(T, H, V, bursty_mask(T, 5), split=1024, seed=12, mode=mode)


def test_fp8_dense_fallback_matches_spans_when_all_active():
    T, H, V = 777, 128, 2600
    mask = np.ones(T, np.uint8)
    r1 = run_fp8(T, H, V, mask, split=1024, seed=13)
    r2 = run_fp8(T, H, V, mask, split=1024, seed=13, use_meta=False)
    assert torch.equal(r1["dH"], r2["dH"]) and torch.equal(r1["dW"], r2["dW"])


def test_fp8_dense_fallback_with_mask():
    T, H, V = 640, 192, 1500
    run_fp8(T, H, V, bursty_mask(T, 7), split=512, seed=14, use_meta=False)


def test_fp8_no_active_token_gives_exact_zero():
    dev = cuda_device()
    T, H, V = 300, 64, 900
    announce("fp8: all inactive")
    hc, s_h, Wc, s_w, y = make_tensors_fp8(T, H, V, 15)
    h, W, y = hc.to(dev), Wc.to(dev), y.to(dev)
    m = torch.zeros(T, dtype=torch.uint8, device=dev)
    lp, ent, lse = flh_forward_fp8(h, s_h, W, s_w, y)
    meta = flh_spans_build(m)
    g = torch.zeros(T, dtype=torch.float32, device=dev)
    dH, dW = flh_backward_fp8(h, s_h, W, s_w, y, lse, ent, g, g, m, meta, 512)
    torch.cuda.synchronize()
    assert not dH.view(torch.int16).any() and float(dW.float().abs().max()) == 0.0


def test_fp8_single_active_token_and_tiny_shapes():
    mask = np.zeros(400, np.uint8)
    mask[257] = 1
    run_fp8(400, 64, 1000, mask, split=256, seed=16)
    for (T, H, V) in [(1, 16, 1), (5, 16, 3), (130, 16, 257), (256, 64, 256)]:
        mask = np.ones(T, np.uint8)
        if T > 2:
            mask[1] = 0
        run_fp8(T, H, V, mask, seed=17, check_rows=False)


def test_fp8_skip_options_match_dense_and_oracle():
    """The weight gradient over active tiles (bitwise the dense one) and the forward over
    active tiles (the oracle's values on active tiles, exactly 0 elsewhere)."""
    T, H, V = 1000, 272, 4000
    mask = bursty_mask(T, 21)
    r_dense = run_fp8(T, H, V, mask, split=2048, seed=23)
    r_skip = run_fp8(T, H, V, mask, split=2048, seed=23, skip_dw=True)
    assert torch.equal(r_dense["dH"], r_skip["dH"]) and torch.equal(r_dense["dW"], r_skip["dW"])
    sp = flh_forward_fp8(r_dense["h"], r_dense["s_h"], r_dense["W"], r_dense["s_w"], r_dense["y"],
                         meta=r_dense["meta"], skip_inactive=True)
    torch.cuda.synchronize()
    tiles = np.zeros(-(-T // 128), bool)
    tiles[np.nonzero(mask)[0] // 128] = True
    in_act = np.repeat(tiles, 128)[:T]
    hc, s_h, Wc, s_w, y = make_tensors_fp8(T, H, V, 23)
    ref = F.forward(hc.numpy(), s_h, Wc.numpy(), s_w, y.numpy())
    for got, dense, o in zip(sp, (r_dense["lp"], r_dense["ent"], r_dense["lse"]), ref):
        g = got.cpu().numpy()
        assert max_abs(g[in_act], o[in_act]) <= TOL_LP and not g[~in_act].any()
        assert np.array_equal(g[in_act], dense.cpu().numpy()[in_act])


def test_fp8_run_to_run_bit_identical():
    T, H, V = 900, 256, 4000
    mask = bursty_mask(T, 9)
    r1 = run_fp8(T, H, V, mask, split=2048, seed=18)
    r2 = run_fp8(T, H, V, mask, split=2048, seed=18)
    for k in ("lp", "ent", "lse", "dH", "dW"):
        assert torch.equal(r1[k], r2[k]), k


def test_fp8_full_size_llama_head_spot_checks():
    """The Llama-3-8B-like head in fp8 at full T, H, V: forward outputs and d_hidden rows
    on sampled tokens against the oracle's per-token definitions (exact at any T),
    inactive rows +0, and the d_weight identities sum_v dW[v, :] = 0 and
    <dH, h> = <dW, W> (h, W the dequantized values).  (Written out here; the stress-head
    check below shares the steps through _fp8_full_size_checks.)"""
    from oracle import lmhead as O
    cfg = CONFIGS[2]
    dev = cuda_device()
    mask, _ = make_mask(2)
    T, H, V = cfg.T, cfg.H, cfg.V
    announce(f"fp8 full size T={T} H={H} V={V}")
    hc, s_h, Wc, s_w, y = make_tensors_fp8(T, H, V, cfg.seed, device=dev)
    a, b = make_upstream(mask)
    m_dev = torch.as_tensor(mask).to(dev)
    meta = flh_spans_build(m_dev)
    lp, ent, lse = flh_forward_fp8(hc, s_h, Wc, s_w, y)
    dH, dW = flh_backward_fp8(hc, s_h, Wc, s_w, y, lse, ent, torch.as_tensor(a).to(dev), torch.as_tensor(b).to(dev),
                              m_dev, meta, cfg.vocab_split)
    torch.cuda.synchronize()
    rng = np.random.default_rng(2)
    act = np.nonzero(mask)[0]
    rows = np.unique(np.concatenate([[0, T - 1, 127, 128], rng.choice(act, 96, replace=False),
                                     rng.integers(0, T, 64)]))
    Wf = F.dequantize(Wc.cpu().numpy(), s_w)
    hr = F.dequantize(hc[torch.as_tensor(rows, device=dev)].cpu().numpy(), s_h)
    yr = y.cpu().numpy()[rows]
    olp, oent, olse = O.forward(hr, Wf, yr)
    assert max_abs(lp.cpu().numpy()[rows], olp) <= TOL_LP
    assert max_abs(ent.cpu().numpy()[rows], oent) <= TOL_LP
    assert max_abs(lse.cpu().numpy()[rows], olse) <= TOL_LP
    ar = rows[mask[rows] != 0]
    sel = np.searchsorted(rows, ar)
    odH = O.dhidden_rows(hr[sel], Wf, yr[sel], mask[ar], a[ar], b[ar], range(len(ar)))
    assert rel_fro(host64(dH[torch.as_tensor(ar, device=dev)]), odH) <= TOL_GRAD
    del Wf
    assert not dH.view(torch.int16)[torch.as_tensor(mask == 0, device=dev)].any()
    dW64 = dW.double()
    col_sum, col_abs = dW64.sum(dim=0), dW64.abs().sum(dim=0)
    assert float((col_sum.abs() / col_abs.clamp_min(1e-300)).max()) <= 1e-2
    h_val = hc.view(torch.float8_e4m3fn).double() * s_h
    W_val = Wc.view(torch.float8_e4m3fn).double() * s_w
    lhs = float((dH.double() * h_val).sum())
    rhs = float((dW64 * W_val).sum())
    assert abs(lhs - rhs) <= 1e-2 * max(abs(lhs), abs(rhs)), (lhs, rhs)


def _fp8_full_size_checks(cid, frac):
    from oracle import lmhead as O
    cfg = CONFIGS[cid]
    dev = cuda_device()
    mask, _ = make_mask(cid, active_frac=frac)
    T, H, V = cfg.T, cfg.H, cfg.V
    announce(f"fp8 full size config {cid} T={T} H={H} V={V} active={mask.mean():.3f}")
    hc, s_h, Wc, s_w, y = make_tensors_fp8(T, H, V, cfg.seed, device=dev)
    a, b = make_upstream(mask)
    m_dev = torch.as_tensor(mask).to(dev)
    meta = flh_spans_build(m_dev)
    lp, ent, lse = flh_forward_fp8(hc, s_h, Wc, s_w, y)
    dH, dW = flh_backward_fp8(hc, s_h, Wc, s_w, y, lse, ent, torch.as_tensor(a).to(dev), torch.as_tensor(b).to(dev),
                              m_dev, meta, cfg.vocab_split)
    torch.cuda.synchronize()
    rng = np.random.default_rng(cid)
    act = np.nonzero(mask)[0]
    rows = np.unique(np.concatenate([[0, T - 1, 127, 128, T - 129], rng.choice(act, 96, replace=False),
                                     rng.integers(0, T, 64)]))
    Wf = F.dequantize(Wc.cpu().numpy(), s_w)
    hr = F.dequantize(hc[torch.as_tensor(rows, device=dev)].cpu().numpy(), s_h)
    yr = y.cpu().numpy()[rows]
    olp, oent, olse = O.forward(hr, Wf, yr)
    assert max_abs(lp.cpu().numpy()[rows], olp) <= TOL_LP
    assert max_abs(ent.cpu().numpy()[rows], oent) <= TOL_LP
    assert max_abs(lse.cpu().numpy()[rows], olse) <= TOL_LP
    ar = rows[mask[rows] != 0]
    sel = np.searchsorted(rows, ar)
    odH = O.dhidden_rows(hr[sel], Wf, yr[sel], mask[ar], a[ar], b[ar], range(len(ar)))
    assert rel_fro(host64(dH[torch.as_tensor(ar, device=dev)]), odH) <= TOL_GRAD
    del Wf
    assert not dH.view(torch.int16)[torch.as_tensor(mask == 0, device=dev)].any()
    dW64 = dW.double()
    col_sum, col_abs = dW64.sum(dim=0), dW64.abs().sum(dim=0)
    assert float((col_sum.abs() / col_abs.clamp_min(1e-300)).max()) <= 1e-2
    lhs = float((dH.double() * (hc.view(torch.float8_e4m3fn).double() * s_h)).sum())
    rhs = float((dW64 * (Wc.view(torch.float8_e4m3fn).double() * s_w)).sum())
    assert abs(lhs - rhs) <= 1e-2 * max(abs(lhs), abs(rhs)), (lhs, rhs)


def test_fp8_full_size_stress_head_spot_checks():
    """The stress head at 50% active in fp8 (the `bench.py --dtype fp8` workload): sampled
    forward outputs and d_hidden rows against the oracle, inactive rows +0, d_weight
    identities."""
    _fp8_full_size_checks(5, 0.5)


def test_fp8_full_size_skip_options_match_dense():
    """The stress head at 50% in fp8: the forward over active tiles gives the dense forward's
    outputs bitwise on active tiles and 0 elsewhere, and the weight gradient over active
    tiles the dense mode's d_hidden and d_weight bitwise."""
    cfg = CONFIGS[5]
    dev = cuda_device()
    mask, _ = make_mask(5, active_frac=0.5)
    T, H, V = cfg.T, cfg.H, cfg.V
    announce(f"fp8 full size skip options T={T} H={H} V={V}")
    hc, s_h, Wc, s_w, y = make_tensors_fp8(T, H, V, cfg.seed, device=dev)
    a, b = make_upstream(mask)
    g_lp, g_ent = torch.as_tensor(a).to(dev), torch.as_tensor(b).to(dev)
    m_dev = torch.as_tensor(mask).to(dev)
    meta = flh_spans_build(m_dev)
    dense = flh_forward_fp8(hc, s_h, Wc, s_w, y)
    sparse = flh_forward_fp8(hc, s_h, Wc, s_w, y, meta=meta, skip_inactive=True)
    torch.cuda.synchronize()
    tiles = np.zeros(-(-T // 128), bool)
    tiles[np.nonzero(mask)[0] // 128] = True
    act = torch.as_tensor(np.repeat(tiles, 128)[:T]).to(dev)
    for d, sp in zip(dense, sparse):
        assert torch.equal(d[act], sp[act]) and not sp[~act].any()
    lp, ent, lse = dense
    del sparse
    dH, dW = flh_backward_fp8(hc, s_h, Wc, s_w, y, lse, ent, g_lp, g_ent, m_dev, meta, cfg.vocab_split)
    dH2, dW2 = flh_backward_fp8(hc, s_h, Wc, s_w, y, lse, ent, g_lp, g_ent, m_dev, meta, cfg.vocab_split,
                                skip_inactive_dw=True)
    torch.cuda.synchronize()
    assert torch.equal(dH, dH2) and torch.equal(dW, dW2)


@pytest.mark.parametrize("cid,frac", [(2, None), (3, None), (4, None), (5, 0.25)])
def test_fp8_full_hv_t_slice_against_oracle(cid, frac):
    """1024-token slices at full H and V in fp8, every output against the oracle."""
    cfg = CONFIGS[cid]
    dev = cuda_device()
    L = 1024
    mask_full, _ = make_mask(cid, active_frac=frac)
    c = np.concatenate([[0], np.cumsum(mask_full, dtype=np.int64)])
    starts = np.arange(0, len(mask_full) - L + 1, 64)
    t0 = int(starts[np.argmin(np.abs((c[starts + L] - c[starts]) / L - 0.5))])
    mask = np.ascontiguousarray(mask_full[t0:t0 + L])
    announce(f"fp8 T-slice config {cid} tokens [{t0}, {t0 + L}) H={cfg.H} V={cfg.V}")
    hc_full, s_h, Wc, s_w, y_full = make_tensors_fp8(cfg.T, cfg.H, cfg.V, cfg.seed, device=dev)
    hc = hc_full[t0:t0 + L].contiguous()
    y = y_full[t0:t0 + L].contiguous()
    del hc_full, y_full
    a, b = make_upstream(mask)
    m_dev = torch.as_tensor(mask).to(dev)
    meta = flh_spans_build(m_dev)
    lp, ent, lse = flh_forward_fp8(hc, s_h, Wc, s_w, y)
    dH, dW = flh_backward_fp8(hc, s_h, Wc, s_w, y, lse, ent, torch.as_tensor(a).to(dev), torch.as_tensor(b).to(dev),
                              m_dev, meta, cfg.vocab_split)
    torch.cuda.synchronize()
    hn, Wn, yn = hc.cpu().numpy(), Wc.cpu().numpy(), y.cpu().numpy()
    olp, oent, olse = F.forward(hn, s_h, Wn, s_w, yn)
    assert max_abs(lp.cpu().numpy(), olp) <= TOL_LP
    assert max_abs(ent.cpu().numpy(), oent) <= TOL_LP
    odH, odW = F.backward(hn, s_h, Wn, s_w, yn, mask, a, b)
    gdW = host64(dW)
    assert rel_fro(host64(dH), odH) <= TOL_GRAD
    assert rel_fro(gdW, odW) <= TOL_GRAD and tile_rel_fro(gdW, odW) <= TOL_TILE
    assert not dH.view(torch.int16).cpu().numpy()[mask == 0].any()


def test_fp8_full_size_dweight_every_entry_on_sampled_upstream():
    """The stress head at 50% in fp8: full-size d_weight entry by entry (and tile by tile)
    against the oracle's backward of 256 sampled tokens, the upstream gradients being zero
    elsewhere (tokens enter the loss independently, so that is the whole d_weight);
    d_hidden: the sampled active rows against the oracle, every other row exactly zero."""
    cfg = CONFIGS[5]
    dev = cuda_device()
    mask, _ = make_mask(5, active_frac=0.5)
    T, H, V = cfg.T, cfg.H, cfg.V
    announce(f"fp8 full-size dW, sampled upstream: T={T} H={H} V={V}")
    hc, s_h, Wc, s_w, y = make_tensors_fp8(T, H, V, cfg.seed, device=dev)
    rng = np.random.default_rng(205)
    act_all = np.nonzero(mask)[0]
    rows = np.unique(np.concatenate([rng.choice(act_all, 240, replace=False), [act_all[0], act_all[-1]],
                                     rng.choice(np.nonzero(mask == 0)[0], 14, replace=False)]))
    a_full, b_full = make_upstream(mask)
    a = np.zeros_like(a_full)
    b = np.zeros_like(b_full)
    a[rows], b[rows] = a_full[rows], b_full[rows]
    off = rows[mask[rows] == 0]
    a[off], b[off] = 0.75, -0.5  # nonzero upstream on inactive tokens: the mask must zero it
    m_dev = torch.as_tensor(mask).to(dev)
    meta = flh_spans_build(m_dev)
    lp, ent, lse = flh_forward_fp8(hc, s_h, Wc, s_w, y)
    dH, dW = flh_backward_fp8(hc, s_h, Wc, s_w, y, lse, ent, torch.as_tensor(a).to(dev), torch.as_tensor(b).to(dev),
                              m_dev, meta, cfg.vocab_split)
    torch.cuda.synchronize()
    keep = np.zeros(T, bool)
    keep[rows[mask[rows] != 0]] = True
    assert not bool((dH[torch.as_tensor(~keep, device=dev)] != 0).any())
    hn = hc[torch.as_tensor(rows, device=dev)].cpu().numpy()
    gdH = host64(dH[torch.as_tensor(rows, device=dev)])
    del dH, hc
    odH, odW = F.backward(hn, s_h, Wc.cpu().numpy(), s_w, y.cpu().numpy()[rows], mask[rows], a[rows], b[rows])
    act = mask[rows] != 0
    assert rel_fro(gdH[act], odH[act]) <= TOL_GRAD
    assert not gdH[~act].any()
    gdW = host64(dW)
    del dW
    torch.cuda.empty_cache()
    assert rel_fro(gdW, odW) <= TOL_GRAD
    assert tile_rel_fro(gdW, odW) <= TOL_TILE
