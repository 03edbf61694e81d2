"""Host-side model of the contraction kernels' memory addressing (CPU only).

Mirrors the index arithmetic of entropy_block_sparse_amd/csrc/flh_gemm.hip --
tile bases, per-thread 32-bit offsets, row clamping, the K-tail clamp, the
transposed-block loads and the epilogue stores -- and checks, for every
workgroup tile, K stage and thread, that each 16-byte load and each store lies
inside its buffer.  It computes no part of the method: it is a bounds check run
over tiny and ragged shapes before kernels go to the GPU.  Keep it in step with
the kernel source.
"""

import itertools

import numpy as np
import pytest

from oracle import spans as S

TILE, SKIP, SPAN_TILE = 256, 128, 256
tid = np.arange(256)
lane = tid & 63
wave = tid >> 6
kchunk = lane & 7
U32 = (1 << 32)


def cdiv(a, b):
    return (a + b - 1) // b


class Buf:
    def __init__(self, name, nbytes):
        self.name, self.n = name, int(nbytes)

    def check(self, addr, width, what):
        addr = np.asarray(addr, np.int64)
        bad = (addr < 0) | (addr + width > self.n)
        assert not bad.any(), f"{what}: {self.name} access out of bounds " \
                              f"(min {addr.min()}, max {addr.max() + width}, size {self.n})"
        assert (addr % 4 == 0).all() or width < 4, f"{what}: misaligned {self.name} access"


def _stages(nk, sample):
    return sorted({0, 1, nk - 2, nk - 1} & set(range(nk))) if sample else range(nk)


def _true_offsets_fit(offs):
    assert (np.asarray(offs, np.int64) < U32).all() and (np.asarray(offs, np.int64) >= 0).all()


def load_rows(buf, bases, offs, K, kper, esz, nk, what, sample=False):
    """bases: (base0, base1) byte offsets; offs: [8, 256] uint32 offsets."""
    c = tid & 7
    BK = 128 // esz
    has_tail = K % BK != 0
    _true_offsets_fit(offs)
    for kt in _stages(nk, sample):
        kb = np.full(256, kt * 128, np.int64)
        if has_tail and kt == nk - 1:
            kok = kt * BK + c * kper < K
            clamp = (((K - 1) // kper) * kper * esz - c * 16) % U32
            kb = np.where(kok, kb, clamp)
        for i in range(8):
            rel = (offs[i].astype(np.int64) + kb) % U32
            buf.check((bases[0] if i < 4 else bases[1]) + rel, 16, f"{what} kt={kt} i={i}")


def load_tr(buf, base, offs, ld, K, kper, esz, nk, what, sample=False):
    BK = 128 // esz
    _true_offsets_fit(offs)
    assert 63 * ld + max(np.max(o) for o in offs) < U32
    for kt in _stages(nk, sample):
        bk = base + kt * BK * ld
        krem = K - kt * BK
        for b in range(8 // kper):
            for i in range(kper):
                kl = np.minimum(kchunk * kper + i, krem - 1)
                rel = (offs[b].astype(np.int64) + kl * ld) % U32
                buf.check(bk + rel, 16, f"{what} kt={kt} b={b} i={i}")


def _pick(n, sample):
    return sorted({0, 1, n - 2, n - 1} & set(range(n))) if sample else range(n)


def model(T, H, V, S_split, esz, mask, sample=False):
    kper = 16 // esz
    BK = 128 // esz
    r_base = tid >> 3
    h = Buf("h", T * H * esz)
    W = Buf("W", V * H * esz)
    w_max = min(V, S_split)
    ld_max = cdiv(w_max, kper) * kper
    D = Buf("D", T * ld_max * esz)
    part = Buf("part", cdiv(V, TILE) * T * 16)
    acc = Buf("acc", T * H * 4)
    dW = Buf("dW", V * H * esz)

    # ---- forward ----
    nk = cdiv(H, BK)
    for mi, ni in itertools.product(_pick(cdiv(V, TILE), sample), _pick(cdiv(T, TILE), sample)):
        v0, t0 = mi * TILE, ni * TILE
        va, tb = V - 1 - v0, T - 1 - t0
        ao = np.stack([np.minimum(r_base + 32 * i, va) * H * esz + (tid & 7) * 16 for i in range(8)])
        bo = np.stack([np.minimum(r_base + 32 * i, tb) * H * esz + (tid & 7) * 16 for i in range(8)])
        load_rows(W, (v0 * H * esz,) * 2, ao, H, kper, esz, nk, f"fwd A mi={mi}", sample)
        load_rows(h, (t0 * H * esz,) * 2, bo, H, kper, esz, nk, f"fwd B ni={ni}", sample)
        cols = np.arange(256)
        t = t0 + cols
        part.check((mi * T + t[t < T]) * 16, 16, "fwd part")

    # ---- backward work lists (as the lists kernel builds them) ----
    flags = S.tile_flags(mask, SKIP)
    n_skip = len(flags)
    tile_list = [i for i, f in enumerate(flags) if f] + [i for i, f in enumerate(flags) if not f]
    n_act = sum(flags)
    spans = S.active_spans(mask, 128)
    stiles = S.span_tiles(spans, SPAN_TILE)

    for sp in _pick(cdiv(V, S_split), sample):
        Ws = min(S_split, V - sp * S_split)
        v_base = sp * S_split
        ld_d = cdiv(Ws, kper) * kper
        assert ld_d <= ld_max
        # ---- d-logits ----
        m_tiles = cdiv(ld_d, TILE)
        n_pairs_gemm, n_pairs_all = cdiv(n_act, 2), cdiv(n_skip, 2)
        nk = cdiv(H, BK)
        for mi in _pick(m_tiles, sample):
            v0 = mi * TILE
            assert v0 <= Ws - 1
            va = Ws - 1 - v0
            for ni in _pick(n_pairs_gemm, sample):
                e0, e1 = 2 * ni, 2 * ni + 1
                tile0 = tile_list[e0]
                tile1 = tile_list[e1] if e1 < n_skip else tile0
                ao = np.stack([np.minimum(r_base + 32 * i, va) * H * esz + (tid & 7) * 16
                               for i in range(8)])
                bo = []
                for i in range(8):
                    rl = (r_base + 32 * i) & 127
                    tb = T - 1 - (tile1 if i >= 4 else tile0) * SKIP
                    bo.append(np.minimum(rl, tb) * H * esz + (tid & 7) * 16)
                load_rows(W, ((v_base + v0) * H * esz,) * 2, ao, H, kper, esz, nk, "dlg A", sample)
                load_rows(h, (tile0 * SKIP * H * esz, tile1 * SKIP * H * esz), np.stack(bo), H,
                          kper, esz, nk, "dlg B", sample)
                # epilogue stores: 4 consecutive columns per (lane, i, q)
                for j in range(4):
                    col = (wave & 1) * 128 + j * 32 + (lane & 31)
                    e = 2 * ni + (col >> 7)
                    tl = np.array([tile_list[x] if x < n_skip else -1 for x in e])
                    t = tl * SKIP + (col & 127)
                    tok = (tl >= 0) & (t < T)
                    for i, q in itertools.product(range(4), range(4)):
                        vv = v0 + (wave >> 1) * 128 + i * 32 + q * 8 + (lane >> 5) * 4
                        ok = tok & (vv < ld_d)
                        D.check((t[ok] * ld_d + vv[ok]) * esz, 4 * esz, "dlg store")
            for p in [x + n_pairs_gemm for x in _pick(n_pairs_all - n_pairs_gemm, sample)]:
                c0, c1 = v0, min(v0 + TILE, ld_d)
                chunks = TILE // kper
                idx = np.arange(TILE * chunks)
                row, ch = idx // chunks, idx % chunks
                e = 2 * p + (row >> 7)
                tl = np.array([tile_list[x] if x < n_skip else -1 for x in e])
                t = tl * SKIP + (row & 127)
                col = c0 + ch * kper
                ok = (tl >= 0) & (t < T) & (col < c1)
                D.check((t[ok] * ld_d + col[ok]) * esz, 16, "dlg zero")
        # ---- dHidden over span tiles ----
        nk = cdiv(Ws, BK)
        for (s0, s1), ni in itertools.product([stiles[x] for x in _pick(len(stiles), sample)],
                                              _pick(cdiv(H, TILE), sample)):
            ramax = s1 - 1 - s0
            ao = np.stack([np.minimum(r_base + 32 * i, ramax) * ld_d * esz + (tid & 7) * 16
                           for i in range(8)])
            load_rows(D, (s0 * ld_d * esz,) * 2, ao, Ws, kper, esz, nk, "dh A", sample)
            bo = []
            for b in range(8 // kper):
                n = ni * TILE + ((lane >> 3) + 8 * wave + 32 * b) * kper
                n = np.where(n >= H, 0, n)
                bo.append(n * esz)
            load_tr(W, v_base * H * esz, bo, H * esz, Ws, kper, esz, nk, "dh B", sample)
            for i, r in itertools.product(range(4), range(16)):
                t = s0 + (wave >> 1) * 128 + i * 32 + ((r >> 2) << 3) + ((lane >> 5) << 2) + (r & 3)
                for j in range(4):
                    n = ni * TILE + (wave & 1) * 128 + j * 32 + (lane & 31)
                    ok = (t < s1) & (n < H)
                    acc.check((t[ok] * H + n[ok]) * 4, 4, "dh store")
        # ---- dWeight ----
        nk = cdiv(T, BK)
        for mi, ni in itertools.product(_pick(cdiv(Ws, TILE), sample), _pick(cdiv(H, TILE), sample)):
            ao, bo = [], []
            for b in range(8 // kper):
                mch = (lane >> 3) + 8 * wave + 32 * b
                v = mi * TILE + mch * kper
                ao.append(np.where(v >= ld_d, 0, v) * esz)
                n = ni * TILE + mch * kper
                bo.append(np.where(n >= H, 0, n) * esz)
            load_tr(D, 0, ao, ld_d * esz, T, kper, esz, nk, "dw A", sample)
            load_tr(h, 0, bo, H * esz, T, kper, esz, nk, "dw B", sample)
            for i, r in itertools.product(range(4), range(16)):
                v = mi * TILE + (wave >> 1) * 128 + i * 32 + ((r >> 2) << 3) + ((lane >> 5) << 2) + (r & 3)
                for j in range(4):
                    n = ni * TILE + (wave & 1) * 128 + j * 32 + (lane & 31)
                    ok = (v < Ws) & (n < H)
                    dW.check(((v_base + v[ok]) * H + n[ok]) * esz, esz, "dw store")


SHAPES = [
    (1, 8, 1, 256), (5, 8, 3, 256), (130, 16, 257, 256), (256, 64, 256, 256),
    (1000, 520, 5000, 2048), (700, 256, 3000, 1024), (777, 128, 2600, 1024),
    (300, 64, 900, 512), (400, 64, 1000, 256), (257, 72, 263, 256), (129, 8, 7, 256),
]


@pytest.mark.parametrize("esz", [2, 4])
@pytest.mark.parametrize("T,H,V,S_split", SHAPES)
def test_kernel_addressing_in_bounds(T, H, V, S_split, esz):
    if H % (16 // esz):
        pytest.skip("H not a multiple of 16 bytes")
    rng = np.random.default_rng(T * 7 + V)
    for mask in (np.ones(T, np.uint8), (rng.random(T) < 0.4).astype(np.uint8),
                 np.zeros(T, np.uint8)):
        model(T, H, V, S_split, esz, mask)


@pytest.mark.parametrize("cid", [1, 2, 3, 4, 5])
def test_kernel_addressing_full_workloads_sampled(cid):
    """Boundary tiles and K stages at the full workload shapes (32-bit offsets)."""
    from workloads import CONFIGS, make_mask
    cfg = CONFIGS[cid]
    mask, _ = make_mask(cid, active_frac=0.5 if cid == 5 else None)
    model(cfg.T, cfg.H, cfg.V, cfg.vocab_split, 2 if cfg.dtype == "bf16" else 4, mask, sample=True)


# ---- bf16 path: LDS-direct buffer loads -------------------------------------------
# Every global load of the bf16 kernels goes through a buffer descriptor, and the
# hardware returns zeros for any byte at or past the descriptor's range, so memory
# safety reduces to: each descriptor's [base, base + num_records) lies inside its
# allocation.  LDS accesses must stay inside the ring (kNS stages of 32 KiB).

NS, OPSTAGE = 4, 256 * 64


def _rsrc(buf, base, nbytes, what):
    n = 0 if nbytes <= 0 else min(nbytes, 0xFFFFFFFF)
    if n == 0:
        return
    assert 0 <= base and base + n <= buf.n, f"{what}: descriptor [{base}, {base + n}) outside {buf.name} ({buf.n})"


def model_bf16(T, H, V, S_split, mask, sample=False):
    esz = 2
    h = Buf("h", T * H * esz)
    W = Buf("W", V * H * esz)
    ld_max = cdiv(min(V, S_split), 8) * 8
    D = Buf("D", T * ld_max * esz)
    ldb = H * 2

    def rows(buf, base0, n0, base1, n1, ld, what):
        _rsrc(buf, base0, n0 * ld, what + " half0")
        _rsrc(buf, base1, n1 * ld, what + " half1")

    for mi, ni in itertools.product(_pick(cdiv(V, TILE), sample), _pick(cdiv(T, TILE), sample)):
        v0, t0 = mi * TILE, ni * TILE
        nv, nt = V - v0, T - t0
        rows(W, v0 * ldb, min(nv, 128), (v0 + 128) * ldb, nv - 128, ldb, "fwd A")
        rows(h, t0 * ldb, min(nt, 128), (t0 + 128) * ldb, nt - 128, ldb, "fwd B")
    flags = S.tile_flags(mask, SKIP)
    n_skip = len(flags)
    tile_list = [i for i, f in enumerate(flags) if f] + [i for i, f in enumerate(flags) if not f]
    n_act = sum(flags)
    stiles = S.span_tiles(S.active_spans(mask, 128), SPAN_TILE)
    for sp in _pick(cdiv(V, S_split), sample):
        Ws = min(S_split, V - sp * S_split)
        v_base = sp * S_split
        ld_d = cdiv(Ws, 8) * 8
        for mi in _pick(cdiv(ld_d, TILE), sample):
            v0 = mi * TILE
            nv = Ws - v0
            rows(W, (v_base + v0) * ldb, min(nv, 128), (v_base + v0 + 128) * ldb, nv - 128, ldb, "dlg A")
            for ni in _pick(cdiv(n_act, 2), sample):
                t0 = tile_list[2 * ni]
                t1 = tile_list[2 * ni + 1] if 2 * ni + 1 < n_skip else -1
                n0 = T - t0 * SKIP
                n1 = T - t1 * SKIP if t1 >= 0 else 0
                rows(h, t0 * SKIP * ldb, min(n0, 128), max(t1, 0) * SKIP * ldb, min(n1, 128), ldb, "dlg B")
        nk = cdiv(Ws, 32)
        for (s0, s1) in [stiles[x] for x in _pick(len(stiles), sample)]:
            nr = s1 - s0
            rows(D, s0 * ld_d * 2, min(nr, 128), (s0 + 128) * ld_d * 2, nr - 128, ld_d * 2, "dh A")
        for s in _pick(nk, sample):
            _rsrc(W, (v_base + s * 32) * ldb, (Ws - s * 32) * ldb, f"dh B stage {s}")
        nk = cdiv(T, 32)
        for s in _pick(nk, sample):
            _rsrc(D, s * 32 * ld_d * 2, (T - s * 32) * ld_d * 2, f"dw A stage {s}")
            _rsrc(h, s * 32 * ldb, (T - s * 32) * ldb, f"dw B stage {s}")
    # LDS: direct-load destinations and fragment reads stay inside one stage operand
    for w, n, l in itertools.product(range(4), range(4), range(64)):
        assert (4 * w + n) * 1024 + l * 16 + 16 <= OPSTAGE
        assert (8 * w + 2 * n) * 512 + l * 16 + 16 <= OPSTAGE
    for l in range(64):
        li, g16, h16 = l & 15, l >> 5, (l >> 4) & 1
        for q, i, wb in itertools.product(range(2), range(4), (0, 128)):
            R = wb + 32 * i + (l & 31)
            assert R * 64 + 64 <= OPSTAGE
            m = wb + 32 * i + 16 * h16 + 4 * (li & 3)
            col = (((m >> 3) ^ (4 * ((li >> 2) & 3))) << 4) + ((m & 7) << 1)
            k0 = 16 * q + 8 * g16 + (li >> 2)
            assert (k0 + 4) * 512 + col + 8 <= OPSTAGE


@pytest.mark.parametrize("T,H,V,S_split", SHAPES)
def test_bf16_descriptors_in_bounds(T, H, V, S_split):
    rng = np.random.default_rng(T + 3 * V)
    for mask in (np.ones(T, np.uint8), (rng.random(T) < 0.4).astype(np.uint8), np.zeros(T, np.uint8)):
        model_bf16(T, H, V, S_split, mask)


@pytest.mark.parametrize("cid", [2, 3, 4, 5])
def test_bf16_descriptors_full_workloads_sampled(cid):
    from workloads import CONFIGS, make_mask
    cfg = CONFIGS[cid]
    mask, _ = make_mask(cid, active_frac=0.5 if cid == 5 else None)
    model_bf16(cfg.T, cfg.H, cfg.V, cfg.vocab_split, mask, sample=True)
