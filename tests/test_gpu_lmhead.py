"""Forward and backward of the HIP path against the fp64 oracle, through the C ABI.

Tolerances (bf16 inputs with fp32 accumulation, and fp32 inputs): logprob and
entropy max abs error <= 5e-3; d_hidden and d_weight relative Frobenius error
<= 1e-2.  Exact requirements: d_hidden rows of inactive tokens are bitwise +0;
a loss mask with no active token gives d_hidden = d_weight = 0 exactly; the
dense fallback and the span path agree bit for bit when every token is active;
two runs are bit-identical.  Sources: SkyRL #2376 "Test coverage" (values and
gradients against dense references across partial splits and masks; an
independent fp64 entropy reference) and "How it works".
"""

import numpy as np
import pytest
import torch

from entropy_block_sparse_amd import flh_backward, flh_forward, flh_spans_build
from oracle import lmhead as O
from tests.gpu_common import announce, cuda_device, host64
from tests.helpers import max_abs, rel_fro
from workloads import make_mask, make_tensors, make_upstream

pytestmark = pytest.mark.gpu

TOL_LP = 5e-3
TOL_GRAD = 1e-2
TOL_TILE = 2e-2


def tile_rel_fro(got, ref, tile=256):
    """Largest relative Frobenius error over the tile x tile blocks whose reference is
    not zero."""
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


def run_case(T, H, V, dtype, mask, mode="lp+ent", vocab_split=0, use_meta=True, seed=0,
             check_rows=True, skip_dw=False):
    dev = cuda_device()
    announce(f"lmhead T={T} H={H} V={V} {dtype} mode={mode} split={vocab_split} meta={use_meta} "
             f"skip_dw={skip_dw}")
    h, W, y = make_tensors(T, H, V, dtype, seed, device="cpu")
    h, W, y = h.to(dev), W.to(dev), y.to(dev)
    a, b = make_upstream(mask, mode, seed=seed)
    m_dev = torch.as_tensor(mask).to(dev)
    g_lp = torch.as_tensor(a).to(dev)
    g_ent = None if b is None else torch.as_tensor(b).to(dev)
    lp, ent, lse = flh_forward(h, W, y)
    meta = flh_spans_build(m_dev) if use_meta else None
    dH, dW = flh_backward(h, W, y, lse, ent, g_lp, g_ent, m_dev, meta, vocab_split,
                          skip_inactive_dw=skip_dw)
    torch.cuda.synchronize()

    hh, WW, yy = host64(h), host64(W), y.cpu().numpy()
    olp, oent, olse = O.forward(hh, WW, yy)
    assert max_abs(lp.cpu().numpy(), olp) <= TOL_LP
    assert max_abs(ent.cpu().numpy(), oent) <= TOL_LP
    assert max_abs(lse.cpu().numpy(), olse) <= TOL_LP
    odH, odW = O.backward(hh, WW, yy, mask, a, b)
    gdH, gdW = host64(dH), host64(dW)
    assert rel_fro(gdH, odH) <= TOL_GRAD, rel_fro(gdH, odH)
    assert rel_fro(gdW, odW) <= TOL_GRAD, rel_fro(gdW, odW)
    # every 256 x 256 block of d_weight on its own (a lost or misplaced block fails)
    if mode != "random":
        assert tile_rel_fro(gdW, odW) <= TOL_TILE, tile_rel_fro(gdW, odW)
    inactive = mask == 0
    if inactive.any():
        raw = dH.view(torch.int16 if dtype == "bf16" else torch.int32).cpu().numpy()
        assert not raw[inactive].any(), "inactive d_hidden rows must be bitwise +0"
    if check_rows and (~inactive).any() and mode != "random":
        act = np.nonzero(~inactive)[0]
        # no active row may be silently dropped: each one matches on its own
        num = np.linalg.norm(gdH[act] - odH[act], axis=1)
        den = np.linalg.norm(odH[act], axis=1)
        assert np.all(num <= 3e-2 * den + 1e-12)
    return dict(lp=lp, ent=ent, lse=lse, dH=dH, dW=dW, meta=meta)


def test_tiny_fp32_config():
    mask, _ = make_mask(1)
    r = run_case(512, 256, 4096, "f32", mask, seed=1235)
    # fp32 inputs: the forward is much tighter than the shared bar
    h, W, y = make_tensors(512, 256, 4096, "f32", 1235)
    olp, oent, _ = O.forward(host64(h), host64(W), y.numpy())
    assert max_abs(r["lp"].cpu().numpy(), olp) < 2e-4
    assert max_abs(r["ent"].cpu().numpy(), oent) < 2e-4


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_ragged_multi_split(dtype):
    # T, H, V all ragged: several token tiles with a partial last one, a K tail
    # (H % 64 != 0), three vocabulary splits with a live-width last split of 904.
    T, H, V = 1000, 520, 5000
    mask = bursty_mask(T, 3)
    run_case(T, H, V, dtype, mask, vocab_split=2048, seed=11)


@pytest.mark.parametrize("mode", ["lp", "random"])
def test_upstream_modes(mode):
    T, H, V = 700, 256, 3000
    run_case(T, H, V, "bf16", bursty_mask(T, 5), mode=mode, vocab_split=1024, seed=12)


def test_dense_fallback_matches_spans_when_all_active():
    T, H, V = 777, 128, 2600
    mask = np.ones(T, np.uint8)
    r1 = run_case(T, H, V, "bf16", mask, vocab_split=1024, use_meta=True, seed=13)
    r2 = run_case(T, H, V, "bf16", mask, vocab_split=1024, use_meta=False, seed=13)
    assert torch.equal(r1["dH"], r2["dH"]) and torch.equal(r1["dW"], r2["dW"])


def test_dense_fallback_with_mask():
    T, H, V = 640, 192, 1500
    run_case(T, H, V, "bf16", bursty_mask(T, 7), vocab_split=512, use_meta=False, seed=14)


def test_no_active_token_gives_exact_zero():
    dev = cuda_device()
    T, H, V = 300, 64, 900
    announce("lmhead: all inactive")
    h, W, y = [x.to(dev) for x in make_tensors(T, H, V, "bf16", 15)]
    m = torch.zeros(T, dtype=torch.uint8, device=dev)
    lp, ent, lse = flh_forward(h, W, y)
    meta = flh_spans_build(m)
    g = torch.zeros(T, dtype=torch.float32, device=dev)
    dH, dW = flh_backward(h, W, y, lse, ent, g, g, m, meta, 512)
    assert int(meta.num_spans.item()) == 0
    assert not dH.view(torch.int16).any() and float(dW.float().abs().max()) == 0.0


def test_single_active_token():
    T, H, V = 400, 64, 1000
    mask = np.zeros(T, np.uint8)
    mask[257] = 1
    run_case(T, H, V, "bf16", mask, vocab_split=256, seed=16)


def test_vocab_narrower_than_split_and_tiny_shapes():
    for (T, H, V) in [(1, 8, 1), (5, 8, 3), (130, 16, 257), (256, 64, 256)]:
        mask = np.ones(T, np.uint8)
        if T > 2:
            mask[1] = 0
        run_case(T, H, V, "bf16", mask, seed=17, check_rows=False)


def test_run_to_run_bit_identical():
    T, H, V = 900, 256, 4000
    mask = bursty_mask(T, 9)
    r1 = run_case(T, H, V, "bf16", mask, vocab_split=2048, seed=18)
    r2 = run_case(T, H, V, "bf16", mask, vocab_split=2048, seed=18)
    for k in ("lp", "ent", "lse", "dH", "dW"):
        assert torch.equal(r1[k], r2[k]), k


def test_workload_mask_slices():
    # the config-2 and config-3 mask recipes at reduced T/H/V
    for cid, (T, H, V) in [(2, (3000, 256, 6000)), (3, (2048, 128, 3100)), (4, (4096, 64, 5000))]:
        mask, _ = make_mask(cid, T=T)
        run_case(T, H, V, "bf16", mask, vocab_split=2048, seed=100 + cid)


SKIP_DW_CASES = [
    # dtype, T, H, V, split, mask: ragged T (partial last tile), a K tail, three splits
    # with a live-width tail; a single active token; all active; none active
    ("bf16", 1000, 520, 5000, 2048, "bursty"),
    ("f32", 1000, 520, 5000, 2048, "bursty"),
    ("bf16", 900, 256, 4000, 1024, "single"),
    ("bf16", 777, 128, 2600, 1024, "all"),
    ("bf16", 300, 64, 900, 512, "none"),
]


@pytest.mark.parametrize("dtype,T,H,V,split,kind", SKIP_DW_CASES)
def test_skip_inactive_dw_matches_dense(dtype, T, H, V, split, kind):
    """The weight gradient over active token tiles only (FLH_BWD_SKIP_INACTIVE_DW)
    leaves out products with zero d-logits rows only, and forms the remaining partial
    sums in the same groups and order: d_hidden and d_weight equal the dense mode's
    bitwise, and the oracle within the usual tolerances."""
    if kind == "bursty":
        mask = bursty_mask(T, 21)
    elif kind == "single":
        mask = np.zeros(T, np.uint8)
        mask[513] = 1
    elif kind == "all":
        mask = np.ones(T, np.uint8)
    else:
        mask = np.zeros(T, np.uint8)
    if kind == "none":
        dev = cuda_device()
        announce(f"skip_dw: no active token T={T}")
        h, W, y = [x.to(dev) for x in make_tensors(T, H, V, dtype, 22)]
        m = torch.as_tensor(mask).to(dev)
        lp, ent, lse = flh_forward(h, W, y)
        meta = flh_spans_build(m)
        g = torch.zeros(T, dtype=torch.float32, device=dev)
        out = [flh_backward(h, W, y, lse, ent, g, g, m, meta, split, skip_inactive_dw=s) for s in (False, True)]
        torch.cuda.synchronize()
        assert float(out[1][1].float().abs().max()) == 0.0 and not out[1][0].view(torch.int16).any()
        assert torch.equal(out[0][1], out[1][1])
        return
    r_dense = run_case(T, H, V, dtype, mask, vocab_split=split, seed=23, check_rows=kind != "single")
    r_skip = run_case(T, H, V, dtype, mask, vocab_split=split, seed=23, check_rows=kind != "single",
                      skip_dw=True)
    assert torch.equal(r_dense["dH"], r_skip["dH"])
    assert torch.equal(r_dense["dW"], r_skip["dW"])


@pytest.mark.parametrize("dtype,T,H,V,split,kind", SKIP_DW_CASES)
def test_forward_skip_inactive_matches_dense(dtype, T, H, V, split, kind):
    """The forward over active 128-token tiles only (FLH_FWD_SKIP_INACTIVE): tokens of
    active tiles get the dense forward's outputs bitwise (a token's outputs depend on
    its own logits column only), the others exactly 0, and a backward from these outputs
    equals the one from the dense forward bitwise."""
    dev = cuda_device()
    announce(f"forward skip T={T} H={H} V={V} {dtype} {kind}")
    if kind == "bursty":
        mask = bursty_mask(T, 31)
    elif kind == "single":
        mask = np.zeros(T, np.uint8)
        mask[513] = 1
    elif kind == "all":
        mask = np.ones(T, np.uint8)
    else:
        mask = np.zeros(T, np.uint8)
    h, W, y = [x.to(dev) for x in make_tensors(T, H, V, dtype, 32)]
    m = torch.as_tensor(mask).to(dev)
    meta = flh_spans_build(m)
    dense = flh_forward(h, W, y)
    sparse = flh_forward(h, W, y, meta=meta, skip_inactive=True)
    torch.cuda.synchronize()
    tiles = np.zeros(-(-T // 128), bool)
    tiles[np.nonzero(mask)[0] // 128] = True
    in_active = np.repeat(tiles, 128)[:T]
    act_dev = torch.as_tensor(in_active).to(dev)
    for d, s in zip(dense, sparse):
        assert torch.equal(d[act_dev], s[act_dev])
        assert not s[~act_dev].any()
    # and directly against the oracle: its values on tokens of active tiles, 0 elsewhere
    olp, oent, olse = O.forward(host64(h), host64(W), y.cpu().numpy())
    for got, ref in zip(sparse, (olp, oent, olse)):
        g = got.cpu().numpy()
        assert max_abs(g[in_active], ref[in_active]) <= TOL_LP
        assert not g[~in_active].any()
    a, b = make_upstream(mask)
    g_lp, g_ent = torch.as_tensor(a).to(dev), torch.as_tensor(b).to(dev)
    ref = flh_backward(h, W, y, dense[2], dense[1], g_lp, g_ent, m, meta, split)
    out = flh_backward(h, W, y, sparse[2], sparse[1], g_lp, g_ent, m, meta, split)
    torch.cuda.synchronize()
    assert torch.equal(ref[0], out[0]) and torch.equal(ref[1], out[1])


@pytest.mark.parametrize("T,H,V,split,skip_dw", [(1000, 520, 5000, 2048, False), (777, 128, 2600, 1024, False),
                                                 (1000, 520, 5000, 2048, True), (600, 64, 900, 4096, False)])
def test_padded_tail_probe_matches_live_width(T, H, V, split, skip_dw):
    """The padded-staging baseline (FLH_BWD_PADDED_TAIL: the last split staged and launched
    at the full split width, padding zero) gives the live-width results bitwise: the
    padding adds zero products only and no store outside the live rows."""
    dev = cuda_device()
    announce(f"padded tail T={T} H={H} V={V} split={split} skip_dw={skip_dw}")
    mask = bursty_mask(T, 51)
    h, W, y = [x.to(dev) for x in make_tensors(T, H, V, "bf16", 52)]
    m = torch.as_tensor(mask).to(dev)
    meta = flh_spans_build(m)
    a, b = make_upstream(mask)
    g_lp, g_ent = torch.as_tensor(a).to(dev), torch.as_tensor(b).to(dev)
    lp, ent, lse = flh_forward(h, W, y)
    live = flh_backward(h, W, y, lse, ent, g_lp, g_ent, m, meta, split, skip_inactive_dw=skip_dw)
    padded = flh_backward(h, W, y, lse, ent, g_lp, g_ent, m, meta, split, skip_inactive_dw=skip_dw,
                          padded_tail=True)
    torch.cuda.synchronize()
    assert torch.equal(live[0], padded[0]) and torch.equal(live[1], padded[1])
    # and the padded probe's own results against the oracle
    odH, odW = O.backward(host64(h), host64(W), y.cpu().numpy(), mask, a, b)
    assert rel_fro(host64(padded[0]), odH) <= TOL_GRAD and rel_fro(host64(padded[1]), odW) <= TOL_GRAD
    assert tile_rel_fro(host64(padded[1]), odW) <= TOL_TILE


def test_padded_tail_probe_rejects_fp32():
    from entropy_block_sparse_amd._lib import FlhError
    dev = cuda_device()
    T, H, V = 256, 64, 700
    h, W, y = [x.to(dev) for x in make_tensors(T, H, V, "f32", 53)]
    m = torch.ones(T, dtype=torch.uint8, device=dev)
    meta = flh_spans_build(m)
    lp, ent, lse = flh_forward(h, W, y)
    with pytest.raises(FlhError):
        flh_backward(h, W, y, lse, ent, None, None, m, meta, 256, padded_tail=True)


@pytest.mark.parametrize("masked,use_entropy", [(True, True), (True, False), (False, True)])
def test_autograd_op_against_oracle(masked, use_entropy):
    """fused_lm_head as a torch.autograd.Function (the analogue of the pages' op that
    takes optional spans; Bugbot "Overview"): the loss sum_t (a_t logprob_t + b_t
    entropy_t) differentiated through .backward() gives h.grad and W.grad equal to the
    oracle's d_hidden and d_weight for upstream gradients a and b."""
    from entropy_block_sparse_amd import fused_lm_head
    dev = cuda_device()
    T, H, V = 900, 200, 3100
    announce(f"autograd T={T} H={H} V={V} masked={masked} entropy={use_entropy}")
    mask = bursty_mask(T, 61) if masked else np.ones(T, np.uint8)
    h0, W0, y = make_tensors(T, H, V, "bf16", 62)
    h = h0.to(dev).requires_grad_(True)
    W = W0.to(dev).requires_grad_(True)
    y = y.to(dev)
    a, b = make_upstream(mask, "random", seed=63)
    lp, ent = fused_lm_head(h, W, y, torch.as_tensor(mask).to(dev) if masked else None, vocab_split=1024)
    loss = (lp * torch.as_tensor(a).to(dev)).sum()
    if use_entropy:
        loss = loss + (ent * torch.as_tensor(b).to(dev)).sum()
    loss.backward()
    torch.cuda.synchronize()
    hh, WW, yy = host64(h0), host64(W0), y.cpu().numpy()
    olp, oent, _ = O.forward(hh, WW, yy)
    assert max_abs(lp.detach().cpu().numpy(), olp) <= TOL_LP
    assert max_abs(ent.detach().cpu().numpy(), oent) <= TOL_LP
    odH, odW = O.backward(hh, WW, yy, mask if masked else None, a, b if use_entropy else None)
    assert h.grad.dtype == torch.bfloat16 and W.grad.dtype == torch.bfloat16
    assert rel_fro(host64(h.grad), odH) <= TOL_GRAD
    assert rel_fro(host64(W.grad), odW) <= TOL_GRAD
    assert tile_rel_fro(host64(W.grad), odW) <= TOL_TILE
    if masked:
        assert not h.grad.view(torch.int16).cpu().numpy()[mask == 0].any()


def test_metadata_of_another_mask_gives_nan_rows_not_silent_ones():
    """Metadata built from a different mask than the backward's: the rows of active
    tokens it covers (inside one of its spans and its active tiles) are still right, the
    active tokens it leaves out get NaN rows instead of stale or zero ones, and inactive
    rows stay +0 (Bugbot "Note": wrong spans would silently zero gradients)."""
    dev = cuda_device()
    T, H, V = 1000, 64, 1500
    announce("metadata of another mask")
    built = np.zeros(T, np.uint8)
    built[0:400] = 1
    used = np.zeros(T, np.uint8)
    used[300:700] = 1
    h, W, y = [x.to(dev) for x in make_tensors(T, H, V, "bf16", 71)]
    a, b = make_upstream(used)
    meta = flh_spans_build(torch.as_tensor(built).to(dev))
    lp, ent, lse = flh_forward(h, W, y)
    dH, _ = flh_backward(h, W, y, lse, ent, torch.as_tensor(a).to(dev), torch.as_tensor(b).to(dev),
                         torch.as_tensor(used).to(dev), meta, 512)
    torch.cuda.synchronize()
    g = host64(dH)
    odH, _ = O.backward(host64(h), host64(W), y.cpu().numpy(), used, a, b)
    covered = np.arange(300, 400)
    assert np.isfinite(g[covered]).all()
    assert rel_fro(g[covered], odH[covered]) <= TOL_GRAD
    assert np.isnan(g[400:700]).all()
    raw = dH.view(torch.int16).cpu().numpy()
    assert not raw[used == 0].any()
