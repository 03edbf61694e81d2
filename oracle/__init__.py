"""Plain, slow CPU oracle for the block-sparse fused LM head.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or link
anything in this package: only the tests, the smoke check and the CPU-baseline
leg of the benchmark use it.  It shares no code, tables or helpers with the HIP
library.

Source pages (cited below by short name):

* "SkyRL #2376" -- the pull-request page "perf(megatron): add block-sparse fused
  LM-head backward" (NovaSky-AI/SkyRL #2376).  Its sections are cited by their
  headings: "What does this PR do?", "How it works", "Performance",
  "Test coverage", the Bugbot "Overview", the Gemini "Code Review" suggestion
  and the Greptile "Wide-tail grid exceeds live split" finding.

Modules:

* :mod:`oracle.spans`  -- forward active mask as a tile bitmap, ordered active
  spans coalesced across small gaps, active count.  Pure Python.
* :mod:`oracle.lmhead` -- fused linear log-prob / entropy forward and backward in
  float64 numpy, by the plain definition (blocked over tokens only).
* :mod:`oracle.fp8`    -- OCP E4M3 codes decoded to their values, and the fused LM
  head on FP8 inputs with per-tensor scales (the definition above on the values).
* :mod:`oracle.tiny`   -- the same forward/backward in pure Python with
  ``math.fsum``, for shapes of a few tokens; a second, loop-level rendering of
  the definition used to cross-check the numpy one.

Where the pages are silent the readings taken are listed in the module
docstrings (gap counting, span coordinates, tile bitmap order, entropy in nats,
no ignore-index for targets).
"""

from . import fp8, lmhead, spans, tiny  # noqa: F401
