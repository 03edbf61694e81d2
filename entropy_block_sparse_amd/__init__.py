"""Block-sparse fused LM head for AMD Instinct MI355X (gfx950).

The computation lives in libflh.so (C ABI: include/flh.h, HIP kernels in csrc/);
this package only marshals arguments.  Build the library with
``python -m entropy_block_sparse_amd.build``.
"""

from .ops import (  # noqa: F401
    DEFAULT_MAX_GAP,
    DEFAULT_VOCAB_SPLIT,
    ActiveMetaTensors,
    FusedLMHead,
    flh_abi_version,
    flh_backward,
    flh_backward_fp8,
    flh_forward,
    flh_forward_fp8,
    flh_span_capacity,
    flh_spans_build,
    flh_tile_m,
    flh_workspace_bytes,
    fused_lm_head,
    trace_begin,
    trace_end,
)
from ._lib import FlhError, LIB_PATH  # noqa: F401
