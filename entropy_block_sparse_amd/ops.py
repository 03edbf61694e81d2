"""Python binding of the C ABI: argument marshalling only.

Each function has the name of the C entry point it calls.  PyTorch supplies
device memory (outputs, metadata arrays, workspace) and the current stream;
every step of the computation runs in the HIP kernels of libflh.so.
"""

from __future__ import annotations

import ctypes
from dataclasses import dataclass
from typing import List, Optional, Tuple

import torch

from . import _lib
from ._lib import (FLH_BF16, FLH_BWD_PADDED_TAIL, FLH_BWD_SKIP_INACTIVE_DW, FLH_F32, FLH_FP8_E4M3,
                   FLH_FWD_SKIP_INACTIVE, OP_BACKWARD, OP_FORWARD, ActiveMeta, check, lib)

DEFAULT_MAX_GAP = 128
DEFAULT_VOCAB_SPLIT = 16384


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return FLH_BF16
    if t.dtype == torch.float32:
        return FLH_F32
    raise TypeError(f"unsupported dtype {t.dtype} (bf16 or fp32)")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(dev: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _require_cuda(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("all tensors must be on a HIP device")


def _mask_u8(mask: Optional[torch.Tensor]) -> Optional[torch.Tensor]:
    if mask is None:
        return None
    if mask.dtype == torch.bool:
        mask = mask.view(torch.uint8)
    if mask.dtype != torch.uint8:
        raise TypeError("loss_mask must be bool or uint8")
    return mask.contiguous()


def _f32(t: Optional[torch.Tensor]) -> Optional[torch.Tensor]:
    if t is None:
        return None
    if t.dtype != torch.float32:
        raise TypeError("upstream gradients, lse and entropy are float32")
    return t.contiguous()


def flh_abi_version() -> int:
    return int(lib().flh_abi_version())


def flh_tile_m(dtype: torch.dtype = torch.bfloat16) -> int:
    return int(lib().flh_tile_m(FLH_BF16 if dtype == torch.bfloat16 else FLH_F32))


def flh_span_capacity(T: int, max_gap: int = DEFAULT_MAX_GAP) -> int:
    return int(lib().flh_span_capacity(int(T), int(max_gap)))


def _code_of(dtype: torch.dtype) -> int:
    if dtype == torch.bfloat16:
        return FLH_BF16
    if dtype in (torch.uint8, torch.float8_e4m3fn):
        return FLH_FP8_E4M3
    return FLH_F32


def flh_workspace_bytes(op: int, dtype: torch.dtype, T: int, H: int, V: int,
                        vocab_split: int = 0) -> int:
    """dtype: torch.bfloat16, torch.float32, or torch.uint8 / torch.float8_e4m3fn for
    fp8 (OCP E4M3) inputs."""
    code = _code_of(dtype)
    return int(lib().flh_workspace_bytes(int(op), code, int(T), int(H), int(V), int(vocab_split)))


@dataclass
class ActiveMetaTensors:
    """Device arrays of an flh_active_meta plus the host struct pointing at them."""
    T: int
    max_gap: int
    tile_m: int
    spans: torch.Tensor         # [span_cap, 2] int32
    num_spans: torch.Tensor     # [1] int32
    tile_bits: torch.Tensor     # [words] int32 holding uint32 bit patterns
    active_count: torch.Tensor  # [1] int32
    struct: ActiveMeta

    def host_spans(self) -> List[Tuple[int, int]]:
        n = int(self.num_spans.item())
        return [tuple(x) for x in self.spans[:n].cpu().tolist()]

    def host_bits(self) -> List[int]:
        return [w & 0xFFFFFFFF for w in self.tile_bits.cpu().tolist()]


def flh_spans_build(loss_mask: torch.Tensor, max_gap: int = DEFAULT_MAX_GAP,
                    tile_m: Optional[int] = None, span_cap: Optional[int] = None) -> ActiveMetaTensors:
    """Active metadata (tile bitmap, ordered spans, counts) built on the device."""
    m = _mask_u8(loss_mask)
    _require_cuda(m)
    T = int(m.numel())
    tm = flh_tile_m() if tile_m is None else int(tile_m)
    cap = flh_span_capacity(T, max_gap) if span_cap is None else int(span_cap)
    dev = m.device
    n_tiles = (T + tm - 1) // tm if tm > 0 else 0
    spans = torch.empty((max(cap, 1), 2), dtype=torch.int32, device=dev)
    num = torch.empty(1, dtype=torch.int32, device=dev)
    bits = torch.empty(max((n_tiles + 31) // 32, 1), dtype=torch.int32, device=dev)
    cnt = torch.empty(1, dtype=torch.int32, device=dev)
    st = ActiveMeta(T, int(max_gap), tm, cap, spans.data_ptr(), num.data_ptr(), bits.data_ptr(),
                    cnt.data_ptr())
    check(lib().flh_spans_build(_ptr(m), ctypes.byref(st), None, 0, _stream(dev)), "flh_spans_build")
    return ActiveMetaTensors(T, int(max_gap), tm, spans, num, bits, cnt, st)


def _workspace(nbytes: int, dev) -> torch.Tensor:
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=dev)


def _use_workspace(workspace: Optional[torch.Tensor], need: int, dev) -> Tuple[torch.Tensor, int]:
    """(buffer, size in bytes): the caller's workspace, which must be a contiguous tensor on
    the call's device with at least `need` bytes, or, if None, a new one."""
    if workspace is None:
        ws = _workspace(need, dev)
        return ws, ws.numel()
    if workspace.device != dev or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor on the inputs' device")
    nbytes = workspace.numel() * workspace.element_size()
    if nbytes < need:
        raise ValueError(f"workspace holds {nbytes} bytes, the call needs {need}")
    return workspace, nbytes


def _check_operands(h: torch.Tensor, W: torch.Tensor, targets: torch.Tensor):
    """(T, H, V) of a call, after the checks the C ABI cannot make from plain pointers:
    the kernels would read past a tensor that is shorter than the sizes say."""
    if h.dim() != 2 or W.dim() != 2:
        raise ValueError(f"h and W must be 2-D, got {tuple(h.shape)} and {tuple(W.shape)}")
    if h.dtype != W.dtype:
        raise TypeError(f"h and W must share a dtype, got {h.dtype} and {W.dtype}")
    _dtype_code(h)
    T, H = h.shape
    V = W.shape[0]
    if W.shape[1] != H:
        raise ValueError(f"W has {W.shape[1]} columns, h has {H}")
    if targets.numel() != T:
        raise ValueError(f"targets has {targets.numel()} elements, h has {T} rows")
    return int(T), int(H), int(V)


def _check_len(name: str, t: Optional[torch.Tensor], T: int) -> None:
    if t is not None and t.numel() != T:
        raise ValueError(f"{name} has {t.numel()} elements, expected one per token ({T})")


def flh_forward(h: torch.Tensor, W: torch.Tensor, targets: torch.Tensor,
                workspace: Optional[torch.Tensor] = None, meta: Optional["ActiveMetaTensors"] = None,
                skip_inactive: bool = False):
    """Returns (logprob, entropy, lse), each float32 [T].

    skip_inactive: flh_forward_ex's FLH_FWD_SKIP_INACTIVE (needs meta): the forward over
    active 128-token tiles only; the other tiles' tokens get 0."""
    T, H, V = _check_operands(h, W, targets)
    _require_cuda(h, W, targets)
    h, W = h.contiguous(), W.contiguous()
    targets = targets.to(torch.int64).contiguous()
    dev = h.device
    lp = torch.empty(T, dtype=torch.float32, device=dev)
    ent = torch.empty(T, dtype=torch.float32, device=dev)
    lse = torch.empty(T, dtype=torch.float32, device=dev)
    need = flh_workspace_bytes(OP_FORWARD, h.dtype, T, H, V)
    ws, ws_bytes = _use_workspace(workspace, need, dev)
    if skip_inactive:
        if meta is None:
            raise ValueError("skip_inactive needs the active metadata (flh_spans_build)")
        check(lib().flh_forward_ex(_dtype_code(h), _ptr(h), _ptr(W), _ptr(targets), T, H, V, _ptr(lp),
                                   _ptr(ent), _ptr(lse), ctypes.byref(meta.struct), _ptr(ws), ws_bytes,
                                   _stream(dev), FLH_FWD_SKIP_INACTIVE), "flh_forward_ex")
    else:
        check(lib().flh_forward(_dtype_code(h), _ptr(h), _ptr(W), _ptr(targets), T, H, V, _ptr(lp),
                                _ptr(ent), _ptr(lse), _ptr(ws), ws_bytes, _stream(dev)), "flh_forward")
    return lp, ent, lse


def flh_backward(h: torch.Tensor, W: torch.Tensor, targets: torch.Tensor, lse: torch.Tensor,
                 entropy: torch.Tensor, grad_logprob: Optional[torch.Tensor],
                 grad_entropy: Optional[torch.Tensor], loss_mask: Optional[torch.Tensor] = None,
                 meta: Optional[ActiveMetaTensors] = None, vocab_split: int = 0,
                 workspace: Optional[torch.Tensor] = None, skip_inactive_dw: bool = False,
                 padded_tail: bool = False):
    """Returns (d_hidden [T,H], d_weight [V,H]) in the dtype of h.

    skip_inactive_dw: flh_backward_ex's FLH_BWD_SKIP_INACTIVE_DW (the weight gradient
    over active token tiles only; same result).
    padded_tail: FLH_BWD_PADDED_TAIL, the padded-staging baseline of the live-width split
    (a measurement probe; same result)."""
    T, H, V = _check_operands(h, W, targets)
    for name, t in (("lse", lse), ("entropy", entropy), ("grad_logprob", grad_logprob),
                    ("grad_entropy", grad_entropy), ("loss_mask", loss_mask)):
        _check_len(name, t, T)
    if lse is None or entropy is None:
        raise ValueError("lse and entropy saved by flh_forward are required")
    if meta is not None:
        if loss_mask is None:
            raise ValueError("active metadata needs the loss mask it was built from")
        if meta.T != T:
            raise ValueError(f"active metadata describes {meta.T} tokens, the call has {T}")
    _require_cuda(h, W, targets, lse, entropy, grad_logprob, grad_entropy, loss_mask)
    h, W = h.contiguous(), W.contiguous()
    targets = targets.to(torch.int64).contiguous()
    lse, entropy = _f32(lse), _f32(entropy)
    g_lp, g_ent = _f32(grad_logprob), _f32(grad_entropy)
    m = _mask_u8(loss_mask)
    dev = h.device
    dH = torch.empty((T, H), dtype=h.dtype, device=dev)
    dW = torch.empty((V, H), dtype=h.dtype, device=dev)
    need = flh_workspace_bytes(OP_BACKWARD, h.dtype, T, H, V, vocab_split)
    if need == 0:
        raise ValueError("invalid sizes or vocab_split")
    ws, ws_bytes = _use_workspace(workspace, need, dev)
    mp = ctypes.byref(meta.struct) if meta is not None else None
    flags = (FLH_BWD_SKIP_INACTIVE_DW if skip_inactive_dw else 0) | (FLH_BWD_PADDED_TAIL if padded_tail else 0)
    if flags:
        check(lib().flh_backward_ex(_dtype_code(h), _ptr(h), _ptr(W), _ptr(targets), _ptr(lse),
                                    _ptr(entropy), _ptr(g_lp), _ptr(g_ent), _ptr(m), mp, T, H, V,
                                    int(vocab_split), _ptr(dH), _ptr(dW), _ptr(ws), ws_bytes,
                                    _stream(dev), flags), "flh_backward_ex")
    else:
        check(lib().flh_backward(_dtype_code(h), _ptr(h), _ptr(W), _ptr(targets), _ptr(lse),
                                 _ptr(entropy), _ptr(g_lp), _ptr(g_ent), _ptr(m), mp, T, H, V,
                                 int(vocab_split), _ptr(dH), _ptr(dW), _ptr(ws), ws_bytes,
                                 _stream(dev)), "flh_backward")
    return dH, dW


# ---- fp8 (OCP E4M3) inputs ---------------------------------------------------------

def _codes(t: torch.Tensor, name: str) -> torch.Tensor:
    if t.dtype == torch.float8_e4m3fn:
        t = t.view(torch.uint8)
    if t.dtype != torch.uint8:
        raise TypeError(f"{name} must hold E4M3 codes (uint8 or float8_e4m3fn), got {t.dtype}")
    return t.contiguous()


def _check_operands_fp8(h: torch.Tensor, W: torch.Tensor, targets: torch.Tensor):
    if h.dim() != 2 or W.dim() != 2:
        raise ValueError(f"h and W must be 2-D, got {tuple(h.shape)} and {tuple(W.shape)}")
    T, H = h.shape
    if W.shape[1] != H:
        raise ValueError(f"W has {W.shape[1]} columns, h has {H}")
    if targets.numel() != T:
        raise ValueError(f"targets has {targets.numel()} elements, h has {T} rows")
    return int(T), int(H), int(W.shape[0])


def flh_forward_fp8(h: torch.Tensor, scale_h: float, W: torch.Tensor, scale_w: float, targets: torch.Tensor,
                    workspace: Optional[torch.Tensor] = None, meta: Optional["ActiveMetaTensors"] = None,
                    skip_inactive: bool = False):
    """Forward on fp8 inputs: h = scale_h * value(h codes), W = scale_w * value(W codes)
    (OCP E4M3, per-tensor scales).  Returns (logprob, entropy, lse), float32 [T]."""
    T, H, V = _check_operands_fp8(h, W, targets)
    h, W = _codes(h, "h"), _codes(W, "W")
    _require_cuda(h, W, targets)
    targets = targets.to(torch.int64).contiguous()
    dev = h.device
    lp, ent, lse = (torch.empty(T, dtype=torch.float32, device=dev) for _ in range(3))
    need = flh_workspace_bytes(OP_FORWARD, torch.uint8, T, H, V)
    ws, ws_bytes = _use_workspace(workspace, need, dev)
    if skip_inactive and meta is None:
        raise ValueError("skip_inactive needs the active metadata (flh_spans_build)")
    mp = ctypes.byref(meta.struct) if (skip_inactive and meta is not None) else None
    check(lib().flh_forward_fp8(_ptr(h), float(scale_h), _ptr(W), float(scale_w), _ptr(targets), T, H, V,
                                _ptr(lp), _ptr(ent), _ptr(lse), mp, _ptr(ws), ws_bytes, _stream(dev),
                                FLH_FWD_SKIP_INACTIVE if skip_inactive else 0), "flh_forward_fp8")
    return lp, ent, lse


def flh_backward_fp8(h: torch.Tensor, scale_h: float, W: torch.Tensor, scale_w: float, targets: torch.Tensor,
                     lse: torch.Tensor, entropy: torch.Tensor, grad_logprob: Optional[torch.Tensor],
                     grad_entropy: Optional[torch.Tensor], loss_mask: Optional[torch.Tensor] = None,
                     meta: Optional[ActiveMetaTensors] = None, vocab_split: int = 0,
                     workspace: Optional[torch.Tensor] = None, skip_inactive_dw: bool = False):
    """Backward on fp8 inputs: (d_hidden [T,H], d_weight [V,H]) in bf16, the gradients
    with respect to the dequantized h and W."""
    T, H, V = _check_operands_fp8(h, W, targets)
    for name, t in (("lse", lse), ("entropy", entropy), ("grad_logprob", grad_logprob),
                    ("grad_entropy", grad_entropy), ("loss_mask", loss_mask)):
        _check_len(name, t, T)
    if meta is not None:
        if loss_mask is None:
            raise ValueError("active metadata needs the loss mask it was built from")
        if meta.T != T:
            raise ValueError(f"active metadata describes {meta.T} tokens, the call has {T}")
    h, W = _codes(h, "h"), _codes(W, "W")
    _require_cuda(h, W, targets, lse, entropy, grad_logprob, grad_entropy, loss_mask)
    targets = targets.to(torch.int64).contiguous()
    lse, entropy = _f32(lse), _f32(entropy)
    g_lp, g_ent = _f32(grad_logprob), _f32(grad_entropy)
    m = _mask_u8(loss_mask)
    dev = h.device
    dH = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    dW = torch.empty((V, H), dtype=torch.bfloat16, device=dev)
    need = flh_workspace_bytes(OP_BACKWARD, torch.uint8, T, H, V, vocab_split)
    if need == 0:
        raise ValueError("invalid sizes or vocab_split")
    ws, ws_bytes = _use_workspace(workspace, need, dev)
    mp = ctypes.byref(meta.struct) if meta is not None else None
    check(lib().flh_backward_fp8(_ptr(h), float(scale_h), _ptr(W), float(scale_w), _ptr(targets), _ptr(lse),
                                 _ptr(entropy), _ptr(g_lp), _ptr(g_ent), _ptr(m), mp, T, H, V, int(vocab_split),
                                 _ptr(dH), _ptr(dW), _ptr(ws), ws_bytes, _stream(dev),
                                 FLH_BWD_SKIP_INACTIVE_DW if skip_inactive_dw else 0), "flh_backward_fp8")
    return dH, dW


# ---- tracing -------------------------------------------------------------------

def trace_begin(capacity: int = 4096) -> None:
    check(lib().flh_trace_begin(int(capacity)), "flh_trace_begin")


def trace_end(max_records: int = 4096):
    """Waits for the traced launches; returns [(kernel_name, split, ms), ...]."""
    recs = (_lib.TraceRecord * max_records)()
    n = lib().flh_trace_end(recs, max_records)
    if n < 0:
        raise _lib.FlhError(8, "flh_trace_end")
    out = []
    for i in range(min(n, max_records)):
        r = recs[i]
        out.append((lib().flh_kernel_name(r.kernel_id).decode(), int(r.split), float(r.ms)))
    return out


# ---- autograd ------------------------------------------------------------------

class FusedLMHead(torch.autograd.Function):
    """(logprob, entropy) = fused LM head(h, W, targets); backward through the
    block-sparse path when a loss mask is given."""

    @staticmethod
    def forward(ctx, h, W, targets, loss_mask, max_gap, vocab_split):
        lp, ent, lse = flh_forward(h, W, targets)
        meta = flh_spans_build(loss_mask, max_gap) if loss_mask is not None else None
        ctx.save_for_backward(h, W, targets, lse, ent, _mask_u8(loss_mask) if loss_mask is not None else None)
        ctx.meta = meta
        ctx.vocab_split = vocab_split
        return lp, ent

    @staticmethod
    def backward(ctx, g_lp, g_ent):
        h, W, targets, lse, ent, m = ctx.saved_tensors
        g_lp = None if g_lp is None else g_lp.float().contiguous()
        g_ent = None if g_ent is None else g_ent.float().contiguous()
        dH, dW = flh_backward(h, W, targets, lse, ent, g_lp, g_ent, m, ctx.meta, ctx.vocab_split)
        return dH, dW, None, None, None, None


def fused_lm_head(h: torch.Tensor, W: torch.Tensor, targets: torch.Tensor,
                  loss_mask: Optional[torch.Tensor] = None, max_gap: int = DEFAULT_MAX_GAP,
                  vocab_split: int = 0):
    """Per-token (logprob, entropy) of the LM head h W^T, differentiable in h and W."""
    return FusedLMHead.apply(h, W, targets, loss_mask, max_gap, vocab_split)
