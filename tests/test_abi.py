"""The C-ABI library on the CPU: it loads, exports every entry point that
include/flh.h declares, and rejects bad arguments on the host before any
launch (no GPU is touched: every call here fails validation first)."""

import ctypes
import os
import re

import numpy as np
import pytest

from entropy_block_sparse_amd import _lib
from entropy_block_sparse_amd._lib import ActiveMeta, lib

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "flh.h")

E = {v: k for k, v in _lib.STATUS_NAMES.items()}
FAKE = ctypes.c_void_p(0x10000)      # never dereferenced: validation fails first
FAKE_ODD = ctypes.c_void_p(0x10008)  # not 16-byte aligned


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    return sorted(set(re.findall(r"\b(flh_[a-z0-9_]+)\s*\(", text)))


def test_library_loads_and_exports_every_declared_symbol():
    names = declared_functions()
    assert "flh_spans_build" in names and "flh_forward" in names and "flh_backward" in names
    L = lib()
    for n in names:
        assert hasattr(L, n), n
    assert {n for n, _, _ in _lib.SIGNATURES} == set(names)


def test_abi_version_and_queries():
    L = lib()
    assert L.flh_abi_version() == 1
    assert L.flh_tile_m(1) == 128 and L.flh_tile_m(0) == 128 and L.flh_tile_m(7) == 0
    assert L.flh_span_capacity(16384, 128) == 127
    assert L.flh_span_capacity(262144, 128) == 2017
    assert L.flh_span_capacity(0, 128) == 0 and L.flh_span_capacity(10, -1) == 0
    for s in range(11):
        assert L.flh_status_string(s)


def test_span_capacity_matches_oracle():
    from oracle import spans as S
    L = lib()
    for T in (1, 2, 7, 100, 512, 16384, 65536):
        for G in (0, 1, 5, 47, 128):
            assert L.flh_span_capacity(T, G) == S.span_capacity(T, G)


def test_workspace_sizes():
    L = lib()
    f = L.flh_workspace_bytes
    # forward: one 16-byte softmax state per (256-row vocabulary tile, token), then
    # 256 bytes of counts and the token-tile list (int32 per 128-token tile), each
    # section 256-byte aligned
    def up(x):
        return (x + 255) // 256 * 256
    parts = ((128256 + 255) // 256) * 16384 * 16
    assert f(1, 1, 16384, 4096, 128256, 0) == up(up(parts) + 256 + 4 * (16384 // 128))
    b = f(2, 1, 16384, 4096, 128256, 0)
    assert b >= 16384 * 16384 * 2 + 16384 * 4096 * 4   # staging + fp32 accumulator
    assert f(2, 1, 512, 256, 4096, 0) < f(2, 1, 512, 256, 40960, 0)
    # the staging buffer follows the live width: a vocabulary narrower than the split
    assert f(2, 1, 1000, 64, 1000, 16384) < f(2, 1, 1000, 64, 20000, 16384)
    assert f(0, 1, 100, 64, 100, 0) == 0                 # spans need none
    for bad in [(1, 1, 0, 64, 100, 0), (1, 1, 100, 60, 100, 0), (2, 1, 100, 64, 100, 100),
                (1, 9, 100, 64, 100, 0), (1, 1, 100, 64, 0, 0), (1, 0, 100, 66, 100, 0)]:
        assert f(*bad) == 0, bad


def _meta(T=100, G=128, tm=128, cap=None, spans=FAKE, num=FAKE, bits=FAKE, cnt=FAKE):
    return ActiveMeta(T, G, tm, (T + G + 1) // (G + 2) if cap is None else cap,
                      spans.value if spans else None, num.value if num else None,
                      bits.value if bits else None, cnt.value if cnt else None)


def test_spans_build_validation():
    L = lib()
    call = lambda mask, m: L.flh_spans_build(mask, ctypes.byref(m) if m is not None else None, None, 0, None)
    assert call(None, _meta()) == E["FLH_E_NULL"]
    assert call(FAKE, None) == E["FLH_E_NULL"]
    assert call(FAKE, _meta(spans=None)) == E["FLH_E_NULL"]
    assert call(FAKE, _meta(cnt=None)) == E["FLH_E_NULL"]
    assert call(FAKE, _meta(T=0, cap=0)) == E["FLH_E_SHAPE"]
    assert call(FAKE, _meta(T=1 << 31, cap=10 ** 9)) == E["FLH_E_SHAPE"]
    assert call(FAKE, _meta(T=1 << 24, cap=10 ** 9)) == E["FLH_E_SHAPE"]
    assert call(FAKE, _meta(tm=0)) == E["FLH_E_SHAPE"]
    assert call(FAKE, _meta(G=-1, cap=100)) == E["FLH_E_META"]
    assert call(FAKE, _meta(T=1000, G=0, cap=499)) == E["FLH_E_META"]   # needs 500


def _fwd(dt=1, h=FAKE, W=FAKE, y=FAKE, T=512, H=256, V=4096, lp=FAKE, ent=FAKE, lse=FAKE,
         ws=FAKE, nbytes=1 << 40):
    return lib().flh_forward(dt, h, W, y, T, H, V, lp, ent, lse, ws, nbytes, None)


def test_forward_validation():
    assert _fwd(dt=5) == E["FLH_E_DTYPE"]
    for k in ("h", "W", "y", "lp", "ent", "lse", "ws"):
        assert _fwd(**{k: None}) == E["FLH_E_NULL"], k
    assert _fwd(T=0) == E["FLH_E_SHAPE"]
    assert _fwd(V=0) == E["FLH_E_SHAPE"]
    assert _fwd(T=1 << 31) == E["FLH_E_SHAPE"]
    # 2^24: a wave's 64 rows of the backward's transposed operands (rows of about T
    # elements) would need byte offsets past 2^32
    for k in ("T", "H", "V"):
        assert _fwd(**{k: 1 << 24}) == E["FLH_E_SHAPE"], k
        assert _fwd(**{k: (1 << 24) - 8}, nbytes=100) == E["FLH_E_WORKSPACE"], k  # accepted size
    assert lib().flh_workspace_bytes(2, 1, 1 << 24, 64, 2048, 0) == 0
    assert lib().flh_workspace_bytes(2, 1, (1 << 24) - 8, 64, 2048, 0) > 0
    assert _fwd(H=12) == E["FLH_E_SHAPE"]            # bf16 rows must be 16-byte multiples
    assert _fwd(dt=0, H=6) == E["FLH_E_SHAPE"]
    assert _fwd(h=FAKE_ODD) == E["FLH_E_ALIGN"]
    assert _fwd(W=FAKE_ODD) == E["FLH_E_ALIGN"]
    assert _fwd(ws=ctypes.c_void_p(0x10010)) == E["FLH_E_ALIGN"]
    assert _fwd(nbytes=100) == E["FLH_E_WORKSPACE"]


def _bwd(dt=1, h=FAKE, W=FAKE, y=FAKE, lse=FAKE, ent=FAKE, glp=FAKE, gent=FAKE, mask=FAKE,
         meta="ok", T=512, H=256, V=4096, split=0, dH=FAKE, dW=FAKE, ws=FAKE, nbytes=1 << 40):
    m = _meta(T=512) if meta == "ok" else meta
    mp = ctypes.byref(m) if m is not None else None
    return lib().flh_backward(dt, h, W, y, lse, ent, glp, gent, mask, mp, T, H, V, split,
                              dH, dW, ws, nbytes, None)


def test_backward_validation():
    assert _bwd(dt=3) == E["FLH_E_DTYPE"]
    for k in ("h", "W", "y", "lse", "ent", "dH", "dW", "ws"):
        assert _bwd(**{k: None}) == E["FLH_E_NULL"], k
    assert _bwd(split=100) == E["FLH_E_SHAPE"]            # not a multiple of 256
    assert _bwd(split=-256) == E["FLH_E_SHAPE"]
    assert _bwd(H=0) == E["FLH_E_SHAPE"]
    # metadata must match the call (the page: spans are rejected when the layout
    # changes their coordinates)
    assert _bwd(mask=None) == E["FLH_E_META"]
    assert _bwd(meta=_meta(T=511)) == E["FLH_E_META"]
    assert _bwd(meta=_meta(T=512, tm=64)) == E["FLH_E_META"]
    assert _bwd(meta=_meta(T=512, spans=None)) == E["FLH_E_NULL"]
    # a span list that cannot hold every span of this T would have dropped spans, and a
    # negative gap is no metadata flh_spans_build can build (Bugbot "Note": wrong spans
    # silently zero gradients)
    assert _bwd(meta=_meta(T=512, G=-1, cap=512)) == E["FLH_E_META"]
    assert _bwd(meta=_meta(T=512, G=0, cap=255)) == E["FLH_E_META"]      # needs 256
    assert _bwd(meta=_meta(T=512, G=128, cap=3)) == E["FLH_E_META"]     # needs 4
    assert _bwd(meta=_meta(T=512, G=128, cap=-1)) == E["FLH_E_META"]
    assert _bwd(dH=FAKE_ODD) == E["FLH_E_ALIGN"]
    assert _bwd(dW=FAKE_ODD) == E["FLH_E_ALIGN"]
    assert _bwd(nbytes=1000) == E["FLH_E_WORKSPACE"]


def _fwd_ex(flags, meta="ok", dt=1, T=512, H=256, V=4096, nbytes=1 << 40):
    m = _meta(T=512) if meta == "ok" else meta
    mp = ctypes.byref(m) if m is not None else None
    return lib().flh_forward_ex(dt, FAKE, FAKE, FAKE, T, H, V, FAKE, FAKE, FAKE, mp, FAKE, nbytes, None,
                                flags)


def _bwd_ex(flags, dt=1):
    m = _meta(T=512)
    return lib().flh_backward_ex(dt, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, ctypes.byref(m),
                                 512, 256, 4096, 0, FAKE, FAKE, FAKE, 1 << 40, None, flags)


def test_option_entry_point_validation():
    from entropy_block_sparse_amd._lib import FLH_BWD_PADDED_TAIL, FLH_FWD_SKIP_INACTIVE
    # unknown option bits are refused before anything runs
    assert _fwd_ex(1 << 5) == E["FLH_E_UNSUPPORTED"]
    assert _bwd_ex(1 << 7) == E["FLH_E_UNSUPPORTED"]
    # the forward over active tiles needs metadata of this T and tile height
    assert _fwd_ex(FLH_FWD_SKIP_INACTIVE, meta=None) == E["FLH_E_META"]
    assert _fwd_ex(FLH_FWD_SKIP_INACTIVE, meta=_meta(T=511)) == E["FLH_E_META"]
    assert _fwd_ex(FLH_FWD_SKIP_INACTIVE, meta=_meta(T=512, tm=64)) == E["FLH_E_META"]
    assert _fwd_ex(FLH_FWD_SKIP_INACTIVE, meta=_meta(T=512, bits=None)) == E["FLH_E_NULL"]
    assert _fwd_ex(FLH_FWD_SKIP_INACTIVE, nbytes=1000) == E["FLH_E_WORKSPACE"]
    # the padded-staging probe is bf16 only
    assert _bwd_ex(FLH_BWD_PADDED_TAIL, dt=0) == E["FLH_E_UNSUPPORTED"]


def test_python_binding_names_match_abi():
    import entropy_block_sparse_amd as pkg
    for n in ("flh_spans_build", "flh_forward", "flh_backward", "flh_workspace_bytes",
              "flh_span_capacity", "flh_tile_m", "flh_abi_version"):
        assert callable(getattr(pkg, n))


def test_product_path_does_not_import_oracle():
    pkg_dir = os.path.join(os.path.dirname(HEADER), "..", "entropy_block_sparse_amd")
    for root, _, files in os.walk(pkg_dir):
        for f in files:
            if f.endswith((".py", ".hip", ".cpp", ".h")):
                src = open(os.path.join(root, f)).read()
                assert "import oracle" not in src and "from oracle" not in src, f


def _fwd_na(dt=1, T=512, H=256, V=4096, flags=0, meta="ok", h=FAKE, lp=FAKE):
    m = _meta(T=T) if meta == "ok" else meta
    mp = ctypes.byref(m) if m is not None else None
    return lib().flh_forward_noalloc(dt, h, FAKE, FAKE, T, H, V, lp, FAKE, FAKE, mp, None, flags)


def test_noalloc_forward_validation():
    """The no-allocation forward: the forward's own checks, and sizes whose workspace
    would not fit the library's static scratch refused before anything runs."""
    L = lib()
    cap = 128 << 20
    assert _fwd_na(dt=4) == E["FLH_E_DTYPE"]
    assert _fwd_na(dt=2) == E["FLH_E_UNSUPPORTED"]  # fp8 needs its scales (flh_forward_fp8)
    assert _fwd_na(h=None) == E["FLH_E_NULL"] and _fwd_na(lp=None) == E["FLH_E_NULL"]
    assert _fwd_na(H=12) == E["FLH_E_SHAPE"]
    assert _fwd_na(flags=1 << 4) == E["FLH_E_UNSUPPORTED"]
    assert _fwd_na(flags=1, meta=None) == E["FLH_E_META"]
    assert _fwd_na(h=FAKE_ODD) == E["FLH_E_ALIGN"]
    # at V = 128256 the Llama-3-8B-like head's T = 16384 fits; the largest T is 16743
    assert L.flh_workspace_bytes(1, 1, 16743, 4096, 128256, 0) <= cap
    assert L.flh_workspace_bytes(1, 1, 16744, 4096, 128256, 0) > cap
    assert _fwd_na(T=16744, H=4096, V=128256, meta=None) == E["FLH_E_SCRATCH"]
    assert _fwd_na(T=262144, H=7168, V=129280, meta=None) == E["FLH_E_SCRATCH"]


def _fwd8(sh=0.01, sw=0.001, H=256, T=512, V=4096, h=FAKE, flags=0, meta=None, nbytes=1 << 40):
    mp = ctypes.byref(meta) if meta is not None else None
    return lib().flh_forward_fp8(h, sh, FAKE, sw, FAKE, T, H, V, FAKE, FAKE, FAKE, mp, FAKE, nbytes, None, flags)


def _bwd8(sh=0.01, sw=0.001, H=256, flags=0):
    m = _meta(T=512)
    return lib().flh_backward_fp8(FAKE, sh, FAKE, sw, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, ctypes.byref(m),
                                  512, H, 4096, 0, FAKE, FAKE, FAKE, 1 << 40, None, flags)


def test_fp8_entry_point_validation():
    """fp8 inputs: scales must be finite and positive with a usable product, rows of
    codes whole 16-byte chunks; the generic entry points refuse the fp8 dtype (it needs
    its scales)."""
    L = lib()
    inf = float("inf")
    for sh, sw in ((0.0, 1.0), (-1.0, 1.0), (1.0, inf), (float("nan"), 1.0), (1e-20, 1e-20), (1e20, 1e20)):
        assert _fwd8(sh, sw) == E["FLH_E_SCALE"], (sh, sw)
        assert _bwd8(sh, sw) == E["FLH_E_SCALE"], (sh, sw)
    assert _fwd8(H=24) == E["FLH_E_SHAPE"] and _bwd8(H=24) == E["FLH_E_SHAPE"]   # H % 16
    # a scale product that keeps every logit finite at H = 256 but not at H = 7168
    assert _fwd8(1e15, 1e15, H=7168) == E["FLH_E_SCALE"] and _bwd8(1e15, 1e15, H=7168) == E["FLH_E_SCALE"]
    assert _fwd8(1e15, 1e15, H=256, nbytes=100) == E["FLH_E_WORKSPACE"]
    assert _fwd8(h=None) == E["FLH_E_NULL"]
    assert _fwd8(h=FAKE_ODD) == E["FLH_E_ALIGN"]
    assert _fwd8(flags=1) == E["FLH_E_META"]
    assert _fwd8(nbytes=100) == E["FLH_E_WORKSPACE"]
    assert _bwd8(flags=1 << 6) == E["FLH_E_UNSUPPORTED"]
    assert _fwd(dt=2) == E["FLH_E_UNSUPPORTED"] and _bwd(dt=2) == E["FLH_E_UNSUPPORTED"]
    # workspace: the forward's does not depend on the input dtype; the backward's staging
    # and transposed copies are bf16 for fp8 inputs
    assert L.flh_workspace_bytes(1, 2, 512, 256, 4096, 0) == L.flh_workspace_bytes(1, 1, 512, 256, 4096, 0)
    assert L.flh_workspace_bytes(2, 2, 512, 256, 4096, 0) == L.flh_workspace_bytes(2, 1, 512, 256, 4096, 0)
    assert L.flh_workspace_bytes(1, 2, 512, 24, 4096, 0) == 0 and L.flh_tile_m(2) == 128


def _random_forward_case(rng, dts=(0, 1, 1, 7, 2)):
    """Arguments of flh_forward_ex, each drawn valid or invalid, and the status codes the
    invalid ones map to (the call must return one of them).  An empty set means a valid
    call, which the caller redraws: no call here may pass validation."""
    codes = set()
    dt = int(rng.choice(dts))
    if dt == 7:
        codes.add("FLH_E_DTYPE")
    if dt == 2:
        codes.add("FLH_E_UNSUPPORTED")           # fp8 needs flh_forward_fp8
    flags = int(rng.choice([0, 1, 2, 1 << 5]))
    if flags > 1:
        codes.add("FLH_E_UNSUPPORTED")
    ptr = {}
    for k in ("h", "W", "y", "lp", "ent", "lse"):
        r = rng.random()
        if r < 0.08:
            ptr[k] = None
            codes.add("FLH_E_NULL")
        elif r < 0.16 and k in ("h", "W"):
            ptr[k] = FAKE_ODD
            codes.add("FLH_E_ALIGN")
        else:
            ptr[k] = FAKE
    T = int(rng.choice([1, 300, 4096, 0, -3, 1 << 24]))
    V = int(rng.choice([1, 5000, 5000, 0, 1 << 24]))
    H = int(rng.choice([64, 256, 12, 0, 1 << 24]))
    if T <= 0 or T >= 1 << 24 or V <= 0 or V >= 1 << 24 or H <= 0 or H >= 1 << 24 or (dt == 1 and H % 8):
        codes.add("FLH_E_SHAPE")
    meta = None
    if flags == 1:
        mr = rng.random()
        if mr < 0.15:
            codes.add("FLH_E_META")                # skip needs metadata
        elif mr < 0.3:
            meta = _meta(T=max(T, 1) + 1)
            codes.add("FLH_E_META")                # metadata of another T
        elif mr < 0.4:
            meta = _meta(T=max(T, 1), tm=64)
            codes.add("FLH_E_META")                # another tile height
        elif mr < 0.5:
            meta = _meta(T=max(T, 1), bits=None)
            codes.add("FLH_E_NULL")
        else:
            meta = _meta(T=max(T, 1))
            if T <= 0:
                codes.add("FLH_E_SHAPE")
    ws, nbytes = FAKE, 1 << 40
    wr = rng.random()
    if wr < 0.1:
        ws = None
        codes.add("FLH_E_NULL")
    elif wr < 0.2:
        ws = ctypes.c_void_p(0x10010)
        codes.add("FLH_E_ALIGN")
    elif wr < 0.45:
        nbytes = 100
        codes.add("FLH_E_WORKSPACE")
    args = (dt, ptr["h"], ptr["W"], ptr["y"], T, H, V, ptr["lp"], ptr["ent"], ptr["lse"],
            ctypes.byref(meta) if meta is not None else None, ws, nbytes, None, flags)
    return args, codes


def test_forward_validation_randomised():
    """Random mixes of valid and invalid arguments: every call is rejected before any
    launch with one of the codes its invalid arguments map to (whichever the library
    checks first), never FLH_OK or FLH_E_HIP.  Also runs under the host sanitizers."""
    rng = np.random.default_rng(11)
    L = lib()
    n = 0
    while n < 3000:
        args, codes = _random_forward_case(rng)
        if not codes:
            continue
        st = L.flh_forward_ex(*args)
        assert st in {E[c] for c in codes}, (args, codes, st)
        n += 1


def _random_backward_case(rng, dts=(0, 1, 1, 7, 2)):
    """As _random_forward_case, for flh_backward_ex."""
    codes = set()
    dt = int(rng.choice(dts))
    if dt == 7:
        codes.add("FLH_E_DTYPE")
    if dt == 2:
        codes.add("FLH_E_UNSUPPORTED")
    flags = int(rng.choice([0, 1, 2, 3, 4, 1 << 7]))
    if flags > 3 or (flags & 2 and dt == 0):
        codes.add("FLH_E_UNSUPPORTED")
    ptr = {}
    for k in ("h", "W", "y", "lse", "ent", "dH", "dW"):
        r = rng.random()
        if r < 0.06:
            ptr[k] = None
            codes.add("FLH_E_NULL")
        elif r < 0.12 and k in ("h", "W", "dH", "dW"):
            ptr[k] = FAKE_ODD
            codes.add("FLH_E_ALIGN")
        else:
            ptr[k] = FAKE
    glp = FAKE if rng.random() < 0.8 else None   # optional: NULL is the zero gradient
    gent = FAKE if rng.random() < 0.7 else None
    T = int(rng.choice([1, 300, 4096, 0, -3, 1 << 24]))
    V = int(rng.choice([1, 5000, 5000, 0, 1 << 24]))
    H = int(rng.choice([64, 256, 12, 0, 1 << 24]))
    split = int(rng.choice([0, 256, 16384, 100, -256, 384]))
    if (T <= 0 or T >= 1 << 24 or V <= 0 or V >= 1 << 24 or H <= 0 or H >= 1 << 24 or (dt == 1 and H % 8)
            or split < 0 or split % 256):
        codes.add("FLH_E_SHAPE")
    mask = FAKE
    meta = None
    mr = rng.random()
    if mr < 0.3:
        meta = None                                  # dense fallback; the mask may be NULL
        if rng.random() < 0.5:
            mask = None
    else:
        Tm = max(T, 1)
        if mr < 0.4:
            meta = _meta(T=Tm + 1)
            codes.add("FLH_E_META")
        elif mr < 0.5:
            meta = _meta(T=Tm, tm=64)
            codes.add("FLH_E_META")
        elif mr < 0.58:
            meta = _meta(T=Tm, G=-1, cap=Tm)
            codes.add("FLH_E_META")
        elif mr < 0.66:
            meta = _meta(T=Tm, cap=0)
            codes.add("FLH_E_META")                # a span list that could have dropped spans
        elif mr < 0.74:
            meta = _meta(T=Tm, spans=None)
            codes.add("FLH_E_NULL")
        elif mr < 0.8:
            meta = _meta(T=Tm)
            mask = None
            codes.add("FLH_E_META")                # metadata without its mask
        else:
            meta = _meta(T=Tm)
            if T <= 0:
                codes.add("FLH_E_SHAPE")
    ws, nbytes = FAKE, 1 << 40
    wr = rng.random()
    if wr < 0.08:
        ws = None
        codes.add("FLH_E_NULL")
    elif wr < 0.16:
        ws = ctypes.c_void_p(0x10010)
        codes.add("FLH_E_ALIGN")
    elif wr < 0.4:
        nbytes = 100
        codes.add("FLH_E_WORKSPACE")
    args = (dt, ptr["h"], ptr["W"], ptr["y"], ptr["lse"], ptr["ent"], glp, gent, mask,
            ctypes.byref(meta) if meta is not None else None, T, H, V, split,
            ptr["dH"], ptr["dW"], ws, nbytes, None, flags)
    return args, codes


def test_backward_validation_randomised():
    """As test_forward_validation_randomised, for flh_backward_ex."""
    rng = np.random.default_rng(12)
    L = lib()
    n = 0
    while n < 3000:
        args, codes = _random_backward_case(rng)
        if not codes:
            continue
        st = L.flh_backward_ex(*args)
        assert st in {E[c] for c in codes}, (args, codes, st)
        n += 1


def _random_scales(rng, codes, H):
    """Two fp8 scales, each drawn valid or invalid; FLH_E_SCALE is expected unless both are
    finite and positive with a product in [1e-30, 1e30] that keeps every logit (at most
    448^2 * H code-product units) inside the fp32 range."""
    pool = [0.01, 1.0, 3.5e-3, 0.0, -1.0, float("inf"), float("nan"), 1e-20, 1e20, 1e15, 3e12]
    sh, sw = float(rng.choice(pool)), float(rng.choice(pool))
    ok = (all(x > 0 and x <= 3.0e38 for x in (sh, sw)) and 1e-30 <= sh * sw <= 1e30
          and sh * sw * 448.0 * 448.0 * max(H, 0) < 2.0 ** 127)
    if not ok:
        codes.add("FLH_E_SCALE")
    return sh, sw


def test_fp8_validation_randomised():
    """flh_forward_fp8 and flh_backward_fp8 with random mixes of valid and invalid
    arguments and scales: always rejected before any launch, with an expected code."""
    rng = np.random.default_rng(13)
    L = lib()
    n = 0
    while n < 2000:
        (dt, h, W, y, T, H, V, lp, ent, lse, mp, ws, nb, st, fl), codes = _random_forward_case(rng, dts=(1,))
        sh, sw = _random_scales(rng, codes, H)
        if not codes:
            continue
        s = L.flh_forward_fp8(h, sh, W, sw, y, T, H, V, lp, ent, lse, mp, ws, nb, st, fl)
        assert s in {E[c] for c in codes}, (codes, s)
        n += 1
    n = 0
    while n < 2000:
        a, codes = _random_backward_case(rng, dts=(1,))
        sh, sw = _random_scales(rng, codes, a[11])
        if not codes:
            continue
        s = L.flh_backward_fp8(a[1], sh, a[2], sw, *a[3:])
        assert s in {E[c] for c in codes}, (codes, s)
        n += 1


def test_spans_build_validation_randomised():
    """flh_spans_build with random mixes of valid and invalid arguments: always rejected
    before any launch, with an expected code."""
    rng = np.random.default_rng(14)
    L = lib()
    n = 0
    while n < 2000:
        codes = set()
        mask = FAKE if rng.random() < 0.85 else None
        if mask is None:
            codes.add("FLH_E_NULL")
        T = int(rng.choice([1, 100, 5000, 0, -7, 1 << 24]))
        G = int(rng.choice([0, 5, 128, -1]))
        tm = int(rng.choice([128, 128, 0, -128]))
        ptrs = {k: (FAKE if rng.random() < 0.9 else None) for k in ("spans", "num", "bits", "cnt")}
        if None in ptrs.values():
            codes.add("FLH_E_NULL")
        if T <= 0 or T >= 1 << 24 or tm <= 0:
            codes.add("FLH_E_SHAPE")
        if G < 0:
            codes.add("FLH_E_META")
            cap = 10
        else:
            need = (max(T, 0) + G + 1) // (G + 2)
            cap = need if rng.random() < 0.7 else max(need - 1, -1)
            if cap < need:
                codes.add("FLH_E_META")            # a span list that could drop spans
        meta = None if rng.random() < 0.05 else ActiveMeta(
            T, G, tm, cap, *(p.value if p else None for p in (ptrs["spans"], ptrs["num"], ptrs["bits"], ptrs["cnt"])))
        if meta is None:
            codes = {"FLH_E_NULL"} | ({"FLH_E_NULL"} if mask is None else set())
        if not codes:
            continue
        s = L.flh_spans_build(mask, ctypes.byref(meta) if meta is not None else None, None, 0, None)
        assert s in {E[c] for c in codes}, (T, G, tm, cap, codes, s)
        n += 1
