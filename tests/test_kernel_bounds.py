"""Host-side model of the contraction kernels' memory addressing (CPU only).

Mirrors the index arithmetic of entropy_block_sparse_amd/csrc/flh_gemm.hip and
the transpose in flh_aux.hip -- tile bases, per-thread 32-bit offsets, row
clamping, the K-tail clamp, the bf16 buffer-descriptor ranges and the epilogue
stores -- and checks, for every workgroup tile, K stage and thread, that each
load and each store lies inside its buffer.  It computes no part of the method: it is a bounds check run
over tiny and ragged shapes before kernels go to the GPU.  Keep it in step with
the kernel source.
"""

import itertools

import numpy as np
import pytest

from oracle import spans as S

TILE, SKIP = 256, 128
tid = np.arange(256)
lane = tid & 63
wave = tid >> 6
U32 = (1 << 32)
OPSTAGE = 256 * 128  # bytes of one operand in one stage of the bf16 LDS double buffer


def cdiv(a, b):
    return (a + b - 1) // b


def pad_ld(n):
    """Workspace row stride: a multiple of 64 elements, odd in units of 64."""
    ld = cdiv(n, 64) * 64
    return ld + 64 if (ld // 64) % 2 == 0 else ld


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


def _pick(n, sample):
    return sorted({0, 1, n - 2, n - 1} & set(range(n))) if sample else range(n)


class Src:
    """An operand tile: eight segments of 32 tile rows; segment j is n[j] (0..32) memory
    rows starting at byte offset base[j] of `buf`, ldb bytes apart.  Wave w loads
    segments 2w and 2w+1."""

    def __init__(self, buf, base, n, ldb):
        assert len(base) == len(n) == 8 and all(0 <= x <= 32 for x in n)
        self.buf, self.base, self.n, self.ldb = buf, list(base), list(n), ldb

    @classmethod
    def rows(cls, buf, b, n_rows, ldb):
        """n_rows consecutive rows from byte offset b."""
        return cls(buf, [b + 32 * j * ldb for j in range(8)],
                   [min(max(n_rows - 32 * j, 0), 32) for j in range(8)], ldb)

    @classmethod
    def rows2(cls, buf, b0, n0, b1, n1, ldb):
        """tile rows [0, 128) from b0 (n0 rows), [128, 256) from b1 (n1 rows)."""
        h0, h1 = cls.rows(buf, b0, min(n0, 128), ldb), cls.rows(buf, b1, min(n1, 128), ldb)
        return cls(buf, h0.base[:4] + h1.base[:4], h0.n[:4] + h1.n[:4], ldb)


def load_rows_v1(src, K, esz, what, sample):
    """fp32 path: thread owns chunk (tid & 7) of tile rows (tid >> 3) + 32 i, i.e. row
    tid >> 3 of segment i, clamped onto the segment's last row (an empty segment reads
    segment 0's first row); a chunk wholly past K reads the in-row chunk holding
    element K - 1."""
    kper, BK = 16 // esz, 128 // esz
    nk = cdiv(K, BK)
    r_base = tid >> 3
    c = tid & 7
    offs, bases = [], []
    for i in range(8):
        sg = i if src.n[i] > 0 else 0
        lr = r_base if sg == i else np.zeros(256, np.int64)
        lr = np.minimum(lr, src.n[sg] - 1)
        offs.append(lr * src.ldb + c * 16)
        bases.append(src.base[sg])
    offs = np.stack(offs)
    assert (offs >= 0).all() and (offs < U32).all()
    for kt in _stages(nk, sample):
        kb = np.full(256, kt * 128, np.int64)
        if K % BK and kt == nk - 1:
            inside = kt * BK + c * kper < K
            clamp = (((K - 1) // kper) * kper * esz - c * 16) % U32
            kb = np.where(inside, kb, clamp)
        # every chunk read lies inside its row
        pos = (kb + c * 16) % U32
        assert (pos + 16 <= src.ldb).all(), f"{what} kt={kt}: chunk leaves its row"
        for i in range(8):
            rel = (offs[i] + kb) % U32
            src.buf.check(bases[i] + rel, 16, f"{what} kt={kt} i={i}")


def rsrc_v2(src, K, what):
    """bf16 path: segment j is loaded through a descriptor [base[j], base[j] + n[j] ldb);
    the hardware returns zeros past it, so the range must lie in the buffer."""
    for base, n in zip(src.base, src.n):
        nb = min(n * src.ldb, 0xFFFFFFFF)
        if nb > 0:
            assert 0 <= base and base + nb <= src.buf.n, \
                f"{what}: descriptor [{base}, {base + nb}) outside {src.buf.name} ({src.buf.n})"
    # lane offset (row within the segment, chunk) plus the stage offset fits 32 bits
    assert 31 * src.ldb + 112 + cdiv(K, 64) * 128 < U32, f"{what}: 32-bit offset overflow"


PIECE, PIECES_PER_TILE = 32, 8


def span_pieces(spans, piece=PIECE):
    """Host model of the work-list kernel: each span cut into pieces of at most 32 rows,
    in span order; hidden-gradient tile m takes pieces 8m .. 8m+7."""
    out = []
    for s, e in spans:
        for r in range(s, e, piece):
            out.append((r, min(e, r + piece)))
    return out


def transpose_model(inp, R, C, out, ld_out, esz, what, block=0, tiles=None, esz_in=None):
    """Blocked transpose over 64 x 64 tiles: block b of `block` rows of `in` becomes
    out_b = out + b * C * ld_out, [C][ld_out].  16-byte loads where the vector is whole,
    element loads otherwise; stores likewise.  Gather form (`tiles`: the 128-row tiles
    to take, one block): output column r is input row tiles[r // 128] * 128 + r % 128,
    columns from 128 * len(tiles) on are not written.  Checks bounds and that every
    output element (block, c < C, r < ld_out, or r < 128 * len(tiles)) is written
    exactly once.  esz_in: element size of `in` when it differs (fp8 codes widened to
    bf16): 16-byte loads of 16 // esz_in elements."""
    esz_in = esz_in or esz
    kV = 16 // esz
    kVi = 16 // esz_in
    block = block or R
    n_blocks = cdiv(R, block)
    written = np.zeros((n_blocks, C, ld_out), np.int32)
    for blk in range(n_blocks):
        R_blk = min(block, R - blk * block) if tiles is None else 128 * len(tiles)
        assert tiles is None or 128 * len(tiles) <= ld_out
        for t0 in range(cdiv(ld_out, 64)):
            if tiles is not None and t0 * 64 >= R_blk:
                continue
            for c0t in range(cdiv(C, 64)):
                rb, c0 = t0 * 64, c0t * 64
                idx = np.arange(64 * (64 // kVi))
                rr, cv = idx // (64 // kVi), (idx % (64 // kVi)) * kVi
                r, c = blk * block + rb + rr, c0 + cv
                live = rb + rr < R_blk
                if tiles is not None:
                    src = np.where(live, np.array([tiles[min(x, len(tiles) - 1)] for x in (rb + rr) >> 7]), 0)
                    r = src * 128 + ((rb + rr) & 127)
                    live = live & (r < R)
                whole = live & (c + kVi <= C)
                inp.check((r[whole] * C + c[whole]) * esz_in, 16, what + " load")
                for e in range(kVi):
                    ok = ~whole & live & (c + e < C)
                    inp.check((r[ok] * C + c[ok] + e) * esz_in, esz_in, what + " load1")
                idx = np.arange(64 * (64 // kV))
                cc, rv = idx // (64 // kV), (idx % (64 // kV)) * kV
                c, r = c0 + cc, rb + rv
                live = (c < C) & (r < ld_out)
                whole = live & (r + kV <= ld_out)
                base = blk * C * ld_out
                out.check((base + c[whole] * ld_out + r[whole]) * esz, 16, what + " store")
                for e in range(kV):
                    written[blk, c[whole], r[whole] + e] += 1
                    ok = live & ~whole & (r + e < ld_out)
                    out.check((base + c[ok] * ld_out + r[ok] + e) * esz, esz, what + " store1")
                    written[blk, c[ok], r[ok] + e] += 1
    if tiles is None:
        assert (written == 1).all(), f"{what}: output not covered exactly once"
    else:
        assert (written[:, :, :R_blk] == 1).all() and not written[:, :, R_blk:].any(), what


LS_PITCH, LDS_DLG = 528, 256 * 528  # bf16 d-logits epilogue: LDS tile pitch and size


def dlg_epilogue_v2(D, Dt, pair, T, ld_d, ld_t, t_pad, v0, n_live, n_cols, ni=0, n_act=0, compact=False):
    """bf16 d-logits epilogue: the tile is staged token-major in LDS, then written
    token-major (16-byte chunks of 512-byte rows) and vocabulary-major (transposing
    LDS reads, 16-byte stores)."""
    for j, i in itertools.product(range(8), range(8)):
        col = (wave & 1) * 128 + (lane & 15) + j * 16
        c0 = (wave >> 1) * 128 + (lane >> 4) * 4 + i * 16
        a = col * LS_PITCH + c0 * 2
        assert (a >= 0).all() and (a + 8 <= LDS_DLG).all() and (a % 8 == 0).all()
        # each half-wave of 8-byte writes covers the 64 banks once
        for half in range(2):
            sel = slice(32 * half, 32 * half + 32)
            for w in range(4):
                aw = a[w * 64:(w + 1) * 64][sel]
                banks = {(int(x) // 4 + b) % 64 for x in aw for b in range(2)}
                assert len(banks) == 64
    for k in range(32):
        tl = wave * 64 + 2 * k + (lane >> 5)
        cc = (lane & 31) * 8
        a = tl * LS_PITCH + cc * 2
        assert (a + 16 <= LDS_DLG).all() and (a % 16 == 0).all()
        tile = np.where(tl >> 7, pair[1], pair[0])
        t = tile * SKIP + (tl & 127)
        ok = (tile >= 0) & (t < T) & (cc < n_cols)
        D.check((t[ok] * ld_d + v0 + cc[ok]) * 2, 16, "dlg store (LDS)")
    li, g4 = lane & 15, lane >> 4
    for vb, k in itertools.product(range(4), range(8)):
        mb = wave * 64 + vb * 16
        tb = k * 32 + g4 * 8
        a = (tb + (li >> 2)) * LS_PITCH + (mb + 4 * (li & 3)) * 2
        assert (a % 8 == 0).all() and (a + 4 * LS_PITCH + 8 <= LDS_DLG).all()
        tile = pair[1] if k >> 2 else pair[0]
        t = tile * SKIP + (tb & 127)
        ok = (tile >= 0) & (t < t_pad) & (mb + li < n_live)
        if compact:
            rank = 2 * ni + (k >> 2)
            t = rank * SKIP + (tb & 127)
            ok = (tile >= 0) & (rank < n_act) & (mb + li < n_live)
        Dt.check(((v0 + mb[ok] + li[ok]) * ld_t + t[ok]) * 2, 16, "dlg store^T (LDS)")


def model(T, H, V, S_split, esz, mask, sample=False, compact=False, padded=False, in_esz=None):
    """Walks every (sampled) workgroup tile of the four contractions and checks loads
    (per the fp32 or bf16 load path) and epilogue stores against the buffers.
    in_esz: element size of h and W when it differs from the staging's (fp8 inputs: 1,
    with bf16 staging and transposed copies, esz = 2)."""
    in_esz = in_esz or esz
    kper = 16 // esz
    v2 = esz == 2
    h = Buf("h", T * H * in_esz)
    W = Buf("W", V * H * in_esz)
    w_max = min(V, S_split)
    ld_max = pad_ld(w_max)
    ld_wt, ld_t = pad_ld(w_max), pad_ld(cdiv(T, SKIP) * SKIP)
    t_pad = cdiv(T, kper) * kper  # tokens of the vocabulary-major staging that are written
    D = Buf("D", T * ld_max * esz)
    Dt = Buf("Dt", w_max * ld_t * esz)
    Wt = Buf("Wt", cdiv(V, S_split) * H * ld_wt * esz)
    ht = Buf("ht", H * ld_t * esz)
    part = Buf("part", cdiv(V, TILE) * T * 16)
    acc = Buf("acc", T * H * 4)
    dW = Buf("dW", V * H * esz)

    def loads(src, K, what):
        assert src.n[0] >= 1 or (padded and v2), f"{what}: a tile's first segment always has rows"
        if v2:
            rsrc_v2(src, K, what)
        else:
            load_rows_v1(src, K, esz, what, sample)

    row_q = (wave >> 1) * 128 + (lane >> 4) * 4  # + i*16 + x
    col_q = (wave & 1) * 128 + (lane & 15)        # + j*16

    # ---- forward ----
    ldb = H * in_esz
    for mi, ni in itertools.product(_pick(cdiv(V, TILE), sample), _pick(cdiv(T, TILE), sample)):
        v0, t0 = mi * TILE, ni * TILE
        loads(Src.rows(W, v0 * ldb, V - v0, ldb), H, "fwd A")
        loads(Src.rows(h, t0 * ldb, T - t0, ldb), H, "fwd B")
        t = t0 + np.arange(256)
        part.check((mi * T + t[t < T]) * 16, 16, "fwd part")

    # ---- backward: transposed copies, work lists ----
    if not sample:
        transpose_model(W, V, H, Wt, ld_wt, esz, "W^T", block=S_split, esz_in=in_esz)
    flags = S.tile_flags(mask, SKIP)
    n_skip = len(flags)
    tile_list = [i for i, f in enumerate(flags) if f] + [i for i, f in enumerate(flags) if not f]
    n_act = sum(flags)
    if compact:
        # ---- forward over pairs of active token tiles only (same option run) ----
        for mi, ni in itertools.product(_pick(cdiv(V, TILE), sample), _pick(cdiv(n_act, 2), sample)):
            v0 = mi * TILE
            loads(Src.rows(W, v0 * ldb, V - v0, ldb), H, "fwd-skip A")
            t0 = tile_list[2 * ni]
            t1 = tile_list[2 * ni + 1] if 2 * ni + 1 < n_act else -1
            loads(Src.rows2(h, t0 * SKIP * ldb, T - t0 * SKIP, (t1 if t1 >= 0 else t0) * SKIP * ldb,
                            T - t1 * SKIP if t1 >= 0 else 0, ldb), H, "fwd-skip B")
            for wn_, tl in ((0, t0), (1, t1)):
                if tl < 0:
                    continue
                t = tl * SKIP + np.arange(128)
                part.check((mi * T + t[t < T]) * 16, 16, "fwd-skip part")
    if not sample:
        transpose_model(h, T, H, ht, ld_t, esz, "h^T", tiles=tile_list[:n_act] if compact else None,
                        esz_in=in_esz)
    pieces = span_pieces(S.active_spans(mask, 128))
    dh_tiles = [pieces[PIECES_PER_TILE * m:PIECES_PER_TILE * (m + 1)]
                for m in range(cdiv(len(pieces), PIECES_PER_TILE))]

    for sp in _pick(cdiv(V, S_split), sample):
        Ws = min(S_split, V - sp * S_split)
        v_base = sp * S_split
        Ws_grid = w_max if padded else Ws  # the launches' and the staging's width
        ld_d = pad_ld(Ws_grid)
        w_pad = cdiv(Ws_grid, kper) * kper  # columns of the token-major staging that are written
        assert ld_d <= ld_max and w_pad <= ld_wt and w_pad <= ld_d and t_pad <= ld_t
        # ---- d-logits ----
        m_tiles = cdiv(Ws_grid, TILE)
        n_pairs_gemm, n_pairs_all = cdiv(n_act, 2), cdiv(n_skip, 2)
        for mi in _pick(m_tiles, sample):
            v0 = mi * TILE
            assert v0 <= Ws_grid - 1
            n_live, n_cols = min(Ws - v0, TILE), min(w_pad - v0, TILE)
            wb = (v_base + v0) * ldb
            for ni in _pick(n_pairs_gemm, sample):
                loads(Src.rows(W, wb, Ws - v0, ldb), H, "dlg A")
                t0 = tile_list[2 * ni]
                t1 = tile_list[2 * ni + 1] if 2 * ni + 1 < n_skip else -1
                loads(Src.rows2(h, t0 * SKIP * ldb, T - t0 * SKIP, (t1 if t1 >= 0 else t0) * SKIP * ldb,
                                T - t1 * SKIP if t1 >= 0 else 0, ldb), H, "dlg B")
                pair = (t0, t1)
                if v2:
                    dlg_epilogue_v2(D, Dt, pair, T, ld_d, ld_t, t_pad, v0, n_live, n_cols, ni, n_act, compact)
                    continue
                for j in range(8):
                    col = col_q + j * 16
                    tl = np.array([pair[x] for x in col >> 7])
                    t = tl * SKIP + (col & 127)
                    tok, tokp = (tl >= 0) & (t < T), (tl >= 0) & (t < t_pad)
                    for i in range(8):
                        c0 = row_q + i * 16
                        ok = tok & (c0 < n_cols)
                        D.check((t[ok] * ld_d + v0 + c0[ok]) * esz, 4 * esz, "dlg store")
                        rank = 2 * ni + (col >> 7)
                        tc = rank * SKIP + (col & 127) if compact else t
                        okc = (tl >= 0) & (rank < n_act) if compact else tokp
                        for c in range(4):
                            ok = okc & (c0 + c < n_live)
                            Dt.check(((v0 + c0[ok] + c) * ld_t + tc[ok]) * esz, esz, "dlg store^T")
            for p in [x + n_pairs_gemm for x in _pick(n_pairs_all - n_pairs_gemm, sample)]:
                c1 = min(v0 + TILE, w_pad)
                chunks = TILE // kper
                idx = np.arange(TILE * chunks)
                row, ch = idx // chunks, idx % chunks
                e = 2 * p + (row >> 7)
                tl = np.array([tile_list[x] if x < n_skip else -1 for x in e])
                t = tl * SKIP + (row & 127)
                col = v0 + ch * kper
                ok = (tl >= 0) & (t < T) & (col < c1)
                D.check((t[ok] * ld_d + col[ok]) * esz, 16, "dlg zero")
                vt = SKIP // kper
                idx = np.arange(TILE * 2 * vt)
                vr, rem = idx // (2 * vt), idx % (2 * vt)
                half, vec = rem // vt, rem % vt
                e = 2 * p + half
                v = v0 + vr
                tl = np.array([tile_list[x] if x < n_skip else -1 for x in e])
                t = tl * SKIP + vec * kper
                ok = (tl >= 0) & (v < min(v0 + TILE, Ws)) & (t < t_pad)
                if not compact:  # (the compact layout holds no inactive tile)
                    Dt.check((v[ok] * ld_t + t[ok]) * esz, 16, "dlg zero^T")
        # ---- dHidden over tiles of eight span pieces: A = staging rows, B = W^T rows ----
        ldd, ldw = ld_d * esz, ld_wt * esz
        for tp, ni in itertools.product([dh_tiles[x] for x in _pick(len(dh_tiles), sample)],
                                        _pick(cdiv(H, TILE), sample)):
            ps = [p[0] for p in tp] + [0] * (PIECES_PER_TILE - len(tp))
            pn = [p[1] - p[0] for p in tp] + [0] * (PIECES_PER_TILE - len(tp))
            assert all(1 <= x <= PIECE for x in pn[:len(tp)])
            n0 = ni * TILE
            loads(Src(D, [x * ldd for x in ps], pn, ldd), Ws_grid, "dh A")
            wt = (sp * H + n0) * ldw
            loads(Src.rows(Wt, wt, H - n0, ldw), Ws_grid, "dh B")
            if v2:
                # read-modify-write of whole rows, 16 bytes per lane (4 columns), per
                # 32-row block = one piece
                c4 = lane * 4
                for p, rr in itertools.product(range(2), range(32)):
                    row_b = (wave >> 1) * 128 + (2 * p + (wave & 1)) * 32
                    sg = row_b >> 5
                    tok = np.array([ps[x] for x in sg]) + rr
                    ok = (rr < np.array([pn[x] for x in sg])) & (c4 < min(H - n0, TILE))
                    acc.check((tok[ok] * H + n0 + c4[ok]) * 4, 16, "dh rmw")
                continue
            for i, x in itertools.product(range(8), range(4)):
                row = row_q + i * 16 + x
                sg, lr = row >> 5, row & 31
                t = np.array([ps[x] for x in sg]) + lr
                okr = lr < np.array([pn[x] for x in sg])
                for j in range(8):
                    n = n0 + col_q + j * 16
                    ok = okr & (n < H)
                    acc.check((t[ok] * H + n[ok]) * 4, 4, "dh store")
        # ---- dWeight: A = vocabulary-major staging rows, B = h^T rows ----
        ldt = ld_t * esz
        for mi, ni in itertools.product(_pick(cdiv(Ws_grid, TILE), sample), _pick(cdiv(H, TILE), sample)):
            v0, n0 = mi * TILE, ni * TILE
            K_dw = n_act * SKIP if compact else T
            if K_dw > 0:
                loads(Src.rows(Dt, v0 * ldt, Ws - v0, ldt), K_dw, "dw A")
                loads(Src.rows(ht, n0 * ldt, H - n0, ldt), K_dw, "dw B")
            else:  # nothing to contract: the tile is stored as zeros, 16 bytes per thread
                idx = np.arange(TILE * (TILE // kper))
                r, c = idx // (TILE // kper), (idx % (TILE // kper)) * kper
                ok = (r < min(Ws - v0, TILE)) & (c < min(H - n0, TILE))
                dW.check(((v_base + v0 + r[ok]) * H + n0 + c[ok]) * esz, 16, "dw zero tile")
                continue
            if v2:
                # LDS-staged rows, 16-byte stores (8 columns) via transposing reads
                li, g4 = lane & 15, lane >> 4
                for vb, k in itertools.product(range(4), range(8)):
                    m = wave * 64 + vb * 16 + li
                    cb = k * 32 + g4 * 8
                    ok = (m < min(Ws - v0, TILE)) & (cb < min(H - n0, TILE))
                    dW.check(((v_base + v0 + m[ok]) * H + n0 + cb[ok]) * esz, 16, "dw store (LDS)")
                continue
            for i, x in itertools.product(range(8), range(4)):
                v = v0 + row_q + i * 16 + x
                for j in range(8):
                    n = n0 + col_q + j * 16
                    ok = (v < Ws) & (n < H)
                    dW.check(((v_base + v[ok]) * H + n[ok]) * esz, esz, "dw store")

    if v2:
        # LDS: direct-load destinations (8 lanes per 128-byte row) and fragment reads
        # stay inside one stage operand; the 16 rows a quarter-wave reads together
        # cover all 64 banks
        for w, k, l in itertools.product(range(4), range(8), range(64)):
            row = 64 * w + 8 * k + (l >> 3)
            phys = l & 7
            assert (8 * w + k) * 1024 + l * 16 == row * 128 + phys * 16
            assert (8 * w + k) * 1024 + l * 16 + 16 <= OPSTAGE
        for q, i, wb in itertools.product(range(2), range(8), (0, 128)):
            addrs = []
            for l in range(64):
                R = wb + 16 * i + (l & 15)
                a = R * 128 + ((((4 * q + (l >> 4)) ^ ((R >> 1) & 7))) << 4)
                assert a + 16 <= OPSTAGE
                addrs.append(a)
            for quarter in range(4):
                banks = {((addrs[x] // 4) + b) % 64 for x in range(16 * quarter, 16 * quarter + 16) for b in range(4)}
                assert len(banks) == 64
        if in_esz == 1:
            # fp8 fragments: lane l reads row l % 16, logical chunks 2 (l / 16) and + 1 (the 32
            # bytes at K byte 32 (l / 16)); each of the two reads covers the 64 banks per
            # quarter-wave, and the 8 chunks of a row are read once per fragment
            for i, wb in itertools.product(range(8), (0, 128)):
                seen = set()
                for hh in range(2):
                    addrs = []
                    for l in range(64):
                        R = wb + 16 * i + (l & 15)
                        a = R * 128 + ((((2 * (l >> 4) + hh) ^ ((R >> 1) & 7))) << 4)
                        assert a + 16 <= OPSTAGE
                        addrs.append(a)
                        seen.add(a)
                    for quarter in range(4):
                        banks = {((addrs[x] // 4) + b) % 64 for x in range(16 * quarter, 16 * quarter + 16)
                                 for b in range(4)}
                        assert len(banks) == 64
                assert len(seen) == 16 * 8  # 16 rows x 8 chunks, each once


SHAPES = [
    (1, 8, 1, 256), (5, 8, 3, 256), (130, 16, 257, 256), (256, 64, 256, 256),
    (1000, 520, 5000, 2048), (700, 256, 3000, 1024), (777, 128, 2600, 1024),
    (300, 64, 900, 512), (400, 64, 1000, 256), (257, 72, 263, 256), (129, 8, 7, 256),
]


@pytest.mark.parametrize("T,H,V,S_split", SHAPES)
def test_fp32_addressing_in_bounds(T, H, V, S_split):
    esz = 4
    rng = np.random.default_rng(T * 7 + V)
    for mask in (np.ones(T, np.uint8), (rng.random(T) < 0.4).astype(np.uint8),
                 np.zeros(T, np.uint8)):
        model(T, H, V, S_split, esz, mask)
        model(T, H, V, S_split, esz, mask, compact=True)


FP8_SHAPES = [(1, 16, 1, 256), (130, 16, 257, 256), (1000, 528, 5000, 2048), (777, 128, 2600, 1024),
              (257, 80, 263, 256)]


@pytest.mark.parametrize("T,H,V,S_split", FP8_SHAPES)
def test_fp8_addressing_in_bounds(T, H, V, S_split):
    """fp8 inputs (1-byte codes, H a multiple of 16): the forward and d-logits read the
    codes through the LDS-direct path; staging and transposed copies are bf16."""
    rng = np.random.default_rng(T + V)
    for mask in (np.ones(T, np.uint8), (rng.random(T) < 0.4).astype(np.uint8)):
        model(T, H, V, S_split, 2, mask, in_esz=1)
        model(T, H, V, S_split, 2, mask, compact=True, in_esz=1)


@pytest.mark.parametrize("cid", [1, 2, 3, 4, 5])
def test_kernel_addressing_full_workloads_sampled(cid):
    """Boundary tiles and K stages at the full workload shapes (32-bit offsets)."""
    from workloads import CONFIGS, make_mask
    cfg = CONFIGS[cid]
    mask, _ = make_mask(cid, active_frac=0.5 if cid == 5 else None)
    model(cfg.T, cfg.H, cfg.V, cfg.vocab_split, 2 if cfg.dtype == "bf16" else 4, mask, sample=True)
    model(cfg.T, cfg.H, cfg.V, cfg.vocab_split, 2 if cfg.dtype == "bf16" else 4, mask, sample=True,
          compact=True)
    if cfg.dtype == "bf16":
        model(cfg.T, cfg.H, cfg.V, cfg.vocab_split, 2, mask, sample=True, padded=True)
        model(cfg.T, cfg.H, cfg.V, cfg.vocab_split, 2, mask, sample=True, in_esz=1)


# ---- bf16 path: LDS-direct buffer loads ------------------------------------------------
# Every global load of the bf16 kernels goes through a buffer descriptor, and the hardware
# returns zeros for any byte at or past the descriptor's range, so memory safety of the
# loads reduces to each descriptor's range lying inside its allocation.


@pytest.mark.parametrize("T,H,V,S_split", SHAPES)
def test_bf16_descriptors_in_bounds(T, H, V, S_split):
    rng = np.random.default_rng(T + 3 * V)
    for mask in (np.ones(T, np.uint8), (rng.random(T) < 0.4).astype(np.uint8), np.zeros(T, np.uint8)):
        model(T, H, V, S_split, 2, mask)
        model(T, H, V, S_split, 2, mask, compact=True)
        model(T, H, V, S_split, 2, mask, padded=True)


# ---- tile schedule: XCD-aware remap and grouped rasterization ---------------------------

def _group_map(L, m_tiles, n_tiles, GM):
    per_group = GM * n_tiles
    g = L // per_group
    r = L - g * per_group
    first = g * GM
    gm = min(m_tiles - first, GM)
    return first + r % gm, r // gm


def _tile_of(item, n_gemm, G, m_tiles, n_tiles, GM=8):
    L = item
    if G % 8 == 0:
        r, b = divmod(item, G)
        n_round = min(G, n_gemm - r * G)
        x, q, rem8 = b & 7, n_round >> 3, n_round & 7
        L = r * G + x * q + min(x, rem8) + (b >> 3)
    return _group_map(L, m_tiles, n_tiles, GM)


@pytest.mark.parametrize("m_tiles,n_tiles", [(1, 1), (31, 16), (64, 16), (501, 64), (7, 3), (64, 39), (3, 100)])
@pytest.mark.parametrize("G", [256, 248, 64, 8, 1])
def test_tile_schedule_is_a_bijection(m_tiles, n_tiles, G):
    """Every workgroup tile of a launch is computed exactly once, whatever the grid."""
    n_gemm = m_tiles * n_tiles
    for GM in (8, 4):  # the kernels' group height, and another
        seen = [_tile_of(item, n_gemm, G, m_tiles, n_tiles, GM) for item in range(n_gemm)]
        assert sorted(seen) == [(mi, ni) for mi in range(m_tiles) for ni in range(n_tiles)]
    # with the remap, the tiles one XCD holds in a round are a contiguous run of ids
    if G % 8 == 0 and n_gemm > 8:
        r0 = min(G, n_gemm)
        for x in range(8):
            ids = sorted(_l for _l in [(
                (b & 7) * (r0 >> 3) + min(b & 7, r0 & 7) + (b >> 3)) for b in range(r0) if b & 7 == x])
            assert ids == list(range(ids[0], ids[0] + len(ids))) if ids else True


def test_dhidden_staging_map():
    """bf16 hidden-gradient epilogue: the LDS offsets each wave writes its accumulators
    to and the offsets the storing waves read back name the same (row, column); the
    16 lanes of each 16-byte read fall on distinct banks."""
    DH_GROUP = 4 * 256 + 64
    DH_WAVE = 32 * DH_GROUP
    written = {}
    for w, l, p, ii, j, x in itertools.product(range(4), range(64), range(2), range(4), range(8), range(4)):
        wm, wn, i = w >> 1, w & 1, 4 * p + ii
        row = wm * 128 + i * 16 + 4 * (l >> 4) + x
        col = wn * 128 + j * 16 + (l & 15)
        off = w * DH_WAVE + (ii * 8 + j) * DH_GROUP + x * 256 + l * 4
        assert w * DH_WAVE <= off and off + 4 <= (w + 1) * DH_WAVE <= 4 * DH_WAVE <= 160 * 1024
        assert (p, off) not in written
        written[(p, off)] = (row, col)
    for p, w, rr in itertools.product(range(2), range(4), range(32)):
        rwm, rh = w >> 1, w & 1
        srcs = []
        for l in range(64):
            c4 = l * 4
            lds_col = (c4 >> 7) * DH_WAVE + ((c4 >> 4) & 7) * DH_GROUP + (c4 & 15) * 4
            src = lds_col + rwm * 2 * DH_WAVE + 64 * ((rr & 15) >> 2) + (2 * rh + (rr >> 4)) * 8 * DH_GROUP + (rr & 3) * 256
            assert src % 16 == 0
            for e in range(4):
                assert written[(p, src + 4 * e)] == (rwm * 128 + 64 * p + 32 * rh + rr, c4 + e)
            srcs.append(src)
        for quarter in range(4):
            banks = {(srcs[x] // 4 + b) % 64 for x in range(16 * quarter, 16 * quarter + 16) for b in range(4)}
            assert len(banks) == 64


@pytest.mark.parametrize("seed", range(6))
def test_span_pieces_cover_spans_exactly(seed):
    """The hidden-gradient tiles' pieces cover every span row exactly once, each piece
    lies inside one span and holds 1..32 rows."""
    rng = np.random.default_rng(seed)
    T = int(rng.integers(1, 5000))
    mask = (rng.random(T) < rng.random()).astype(np.uint8)
    spans = S.active_spans(mask, 128)
    pieces = span_pieces(spans)
    covered = np.zeros(T, np.int32)
    for s0, s1 in pieces:
        assert 1 <= s1 - s0 <= PIECE
        assert any(a <= s0 and s1 <= b for a, b in spans)
        covered[s0:s1] += 1
    inside = np.zeros(T, np.int32)
    for a, b in spans:
        inside[a:b] = 1
    assert (covered == inside).all()


def clamped_spans(raw, num, span_cap, T):
    """Host model of how the work-list kernel reads a span list it cannot trust: the
    count clamped to [0, span_cap], each span to 0 <= start <= end <= T."""
    ns = max(0, min(num, span_cap))
    out = []
    for k in range(ns):
        s, e = raw[k]
        s = min(max(s, 0), T)
        e = min(max(e, s), T)
        out.append((s, e))
    return out


@pytest.mark.parametrize("seed", range(6))
def test_span_clamp_keeps_every_piece_inside_the_rows(seed):
    """Metadata that does not belong to the call (another mask, garbage counts or
    coordinates): the pieces the hidden-gradient launch reads and writes stay inside
    [0, T), and at most span_tile_cap of them are stored."""
    rng = np.random.default_rng(seed)
    T = int(rng.integers(1, 3000))
    cap = int(rng.integers(0, 40))
    raw = [(int(rng.integers(-5000, 8000)), int(rng.integers(-5000, 8000))) for _ in range(cap)]
    num = int(rng.integers(-10, 80))
    pieces = span_pieces(clamped_spans(raw, num, cap, T))
    span_tile_cap = cdiv(T, PIECE) + (T + 1) // 2 + 1
    stored = pieces[:span_tile_cap]
    for r0, r1 in stored:
        assert 0 <= r0 < r1 <= T and r1 - r0 <= PIECE
    # the coverage bitmap has one bit per token; its words are indexed below ceil(T/32)
    assert all(t >> 5 < cdiv(T, 32) for t in range(T))
