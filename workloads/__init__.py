"""Seeded synthetic inputs for the fused LM-head tests and benchmark.

This package only draws random numbers (loss masks, hidden states, weights,
targets, upstream gradients).  It holds none of the method's arithmetic and is
the one module that both the oracle-side and the HIP-side of a comparison read
their inputs from.
"""

from .configs import CONFIGS, Config, get_config  # noqa: F401
from .masks import make_mask  # noqa: F401
from .inputs import make_tensors, make_tensors_fp8, make_upstream  # noqa: F401
