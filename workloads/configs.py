"""The five synthetic workloads: shapes, dtypes and mask recipes.

The shapes follow the LM-head shapes the page benchmarks in isolation
(SkyRL #2376, "Performance": four model shapes at 16K-256K tokens, plus a
representative 16K-token shape); the concrete sizes and mask structure are the
ones this project fixes for its own measurements:

1. tiny fp32: T=512 as 4 sequences of 128, H=256, V=4096; first 48 tokens of
   each sequence inactive (prompt).
2. Llama-3-8B-like head, bf16: T=16384, H=4096, V=128256; packed lengths
   U[512, 4096]; prompt prefix 20-60% of each sequence inactive plus random
   inactive gaps of 1-300 tokens in the response; about 45% active.
3. one TP=4 rank's vocabulary share of a 70B-like head, bf16: T=65536, H=8192,
   V=32064; lengths U[1024, 8192]; prompt-prefix masking and short-tail
   responses of 16-256 tokens; about 30% active.
4. Qwen-like wide vocabulary, bf16: T=131072, H=5120, V=152064, vocabulary
   splits of 16384; long responses with gaps <= 128 so spans coalesce; about
   60% active.
5. stress, bf16: T=262144, H=7168, V=129280; alternating active runs (mean 200)
   and gaps (mean 150) thinned or filled to active fractions of 5, 25, 50, 90
   and 100%.
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, Tuple


@dataclass(frozen=True)
class Config:
    cid: int
    name: str
    T: int
    H: int
    V: int
    dtype: str                   # "f32" or "bf16"
    vocab_split: int = 16384
    target_active: float = 0.5   # headline active fraction
    band: float = 0.03           # accepted |achieved - target| for calibration
    sweep: Tuple[float, ...] = field(default_factory=tuple)

    @property
    def seed(self) -> int:
        return 1234 + self.cid


CONFIGS: Dict[int, Config] = {
    1: Config(1, "tiny-fp32 T=512 H=256 V=4096", 512, 256, 4096, "f32",
              target_active=0.625, band=0.0),
    2: Config(2, "llama3-8b-like-head T=16384 H=4096 V=128256", 16384, 4096, 128256, "bf16",
              target_active=0.45, band=0.02),
    3: Config(3, "tp4-70b-like-vocab-share T=65536 H=8192 V=32064", 65536, 8192, 32064, "bf16",
              target_active=0.30, band=0.03),
    4: Config(4, "qwen-like-wide-vocab T=131072 H=5120 V=152064", 131072, 5120, 152064, "bf16",
              target_active=0.60, band=0.02),
    5: Config(5, "stress T=262144 H=7168 V=129280", 262144, 7168, 129280, "bf16",
              target_active=0.50, band=0.03, sweep=(0.05, 0.25, 0.50, 0.90, 1.00)),
}


def get_config(cid: int) -> Config:
    return CONFIGS[int(cid)]
