"""ctypes loader for libflh.so (the C ABI declared in include/flh.h).

The library is built in-tree (``python -m entropy_block_sparse_amd.build``).
If it is missing, importing the ops raises: there is no fallback path.
"""

from __future__ import annotations

import ctypes
import os
import threading

# FLH_LIBRARY names another build of the same ABI (the host-sanitizer build the ABI
# tests load); by default the in-tree library.
LIB_PATH = os.environ.get("FLH_LIBRARY") or os.path.join(os.path.dirname(os.path.abspath(__file__)), "libflh.so")

FLH_OK = 0
STATUS_NAMES = {
    0: "FLH_OK", 1: "FLH_E_NULL", 2: "FLH_E_SHAPE", 3: "FLH_E_DTYPE", 4: "FLH_E_ALIGN",
    5: "FLH_E_WORKSPACE", 6: "FLH_E_META", 7: "FLH_E_UNSUPPORTED", 8: "FLH_E_HIP", 9: "FLH_E_SCRATCH",
    10: "FLH_E_SCALE",
}
FLH_F32, FLH_BF16, FLH_FP8_E4M3 = 0, 1, 2
OP_SPANS, OP_FORWARD, OP_BACKWARD = 0, 1, 2
FLH_BWD_SKIP_INACTIVE_DW = 1  # flh_backward_ex options (include/flh.h)
FLH_BWD_PADDED_TAIL = 2
FLH_FWD_SKIP_INACTIVE = 1  # flh_forward_ex option


class FlhError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = int(status)
        name = STATUS_NAMES.get(self.status, str(status))
        msg = _lib_or_none().flh_status_string(self.status).decode() if _lib_or_none() else ""
        super().__init__(f"{where}: {name} ({msg})")


class ActiveMeta(ctypes.Structure):
    _fields_ = [
        ("T", ctypes.c_int64),
        ("max_gap", ctypes.c_int32),
        ("tile_m", ctypes.c_int32),
        ("span_cap", ctypes.c_int64),
        ("spans", ctypes.c_void_p),
        ("num_spans", ctypes.c_void_p),
        ("tile_bits", ctypes.c_void_p),
        ("active_count", ctypes.c_void_p),
    ]


class TraceRecord(ctypes.Structure):
    _fields_ = [("kernel_id", ctypes.c_int32), ("split", ctypes.c_int32), ("ms", ctypes.c_float)]


# (name, restype, argtypes) of every exported entry point
_VP, _I32, _I64, _SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
SIGNATURES = [
    ("flh_abi_version", _I32, []),
    ("flh_status_string", ctypes.c_char_p, [ctypes.c_int]),
    ("flh_tile_m", _I32, [ctypes.c_int]),
    ("flh_span_capacity", _I64, [_I64, _I32]),
    ("flh_workspace_bytes", _SZ, [ctypes.c_int, ctypes.c_int, _I64, _I64, _I64, _I32]),
    ("flh_spans_build", ctypes.c_int, [_VP, ctypes.POINTER(ActiveMeta), _VP, _SZ, _VP]),
    ("flh_forward", ctypes.c_int,
     [ctypes.c_int, _VP, _VP, _VP, _I64, _I64, _I64, _VP, _VP, _VP, _VP, _SZ, _VP]),
    ("flh_forward_ex", ctypes.c_int,
     [ctypes.c_int, _VP, _VP, _VP, _I64, _I64, _I64, _VP, _VP, _VP, ctypes.POINTER(ActiveMeta), _VP, _SZ,
      _VP, ctypes.c_uint32]),
    ("flh_forward_noalloc", ctypes.c_int,
     [ctypes.c_int, _VP, _VP, _VP, _I64, _I64, _I64, _VP, _VP, _VP, ctypes.POINTER(ActiveMeta), _VP,
      ctypes.c_uint32]),
    ("flh_forward_fp8", ctypes.c_int,
     [_VP, ctypes.c_float, _VP, ctypes.c_float, _VP, _I64, _I64, _I64, _VP, _VP, _VP, ctypes.POINTER(ActiveMeta),
      _VP, _SZ, _VP, ctypes.c_uint32]),
    ("flh_backward_fp8", ctypes.c_int,
     [_VP, ctypes.c_float, _VP, ctypes.c_float, _VP, _VP, _VP, _VP, _VP, _VP, ctypes.POINTER(ActiveMeta),
      _I64, _I64, _I64, _I32, _VP, _VP, _VP, _SZ, _VP, ctypes.c_uint32]),
    ("flh_backward", ctypes.c_int,
     [ctypes.c_int, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, ctypes.POINTER(ActiveMeta),
      _I64, _I64, _I64, _I32, _VP, _VP, _VP, _SZ, _VP]),
    ("flh_backward_ex", ctypes.c_int,
     [ctypes.c_int, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, ctypes.POINTER(ActiveMeta),
      _I64, _I64, _I64, _I32, _VP, _VP, _VP, _SZ, _VP, ctypes.c_uint32]),
    ("flh_trace_begin", ctypes.c_int, [_I32]),
    ("flh_trace_end", _I32, [ctypes.POINTER(TraceRecord), _I32]),
    ("flh_kernel_name", ctypes.c_char_p, [_I32]),
]

_lock = threading.Lock()
_handle = None


def _lib_or_none():
    return _handle


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built."""
    global _handle
    if _handle is not None:
        return _handle
    with _lock:
        if _handle is None:
            if not os.path.exists(LIB_PATH):
                raise ImportError(
                    f"{LIB_PATH} is missing: build it with `python -m entropy_block_sparse_amd.build` "
                    "(the fused LM head has no non-HIP fallback)")
            h = ctypes.CDLL(LIB_PATH)
            for name, res, args in SIGNATURES:
                fn = getattr(h, name)
                fn.restype = res
                fn.argtypes = args
            _handle = h
    return _handle


def check(status: int, where: str) -> None:
    if status != FLH_OK:
        raise FlhError(status, where)
