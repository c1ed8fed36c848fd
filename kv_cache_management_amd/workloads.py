"""The five synthetic R-SWA workloads, with their sizes.

Sizes follow the configuration values of the page "开源5天Star破万之后：百度
Unlimited-OCR的爆火路径复盘" (www.gtnt.cn/news/146005): §2.1 gives the window
W = 128, 32768 positions and about 256 image tokens per 1024x1024 page; §2.2
gives the language hidden size 1280 (split here as 10 heads of 128); §2.4
gives 12 decoder layers.  Inputs are synthetic (see synth.py).
"""

from __future__ import annotations

from dataclasses import dataclass
from typing import Optional, Tuple

import numpy as np

TOKENS_PER_PAGE = 256
WINDOW = 128
MAX_POSITIONS = 32768


@dataclass(frozen=True)
class Workload:
    wid: int
    name: str
    layers: int
    heads: int
    head_dim: int
    dtype: str                      # "bf16" or "f32"
    prefill_lens: Tuple[int, ...]
    window: int
    decode_steps: int
    input_std: float
    rope_base: float = 10000.0
    max_positions: int = MAX_POSITIONS
    # Decode steps each request has already taken before the measured steps
    # (staggered ring phases); None means every request starts at step 0.
    start_steps: Optional[Tuple[int, ...]] = None
    # Page-size-1 pool: logical slot i of a request lives at pool row
    # slot_table[slot_base + i], a shuffled permutation of the pool rows.
    paged: bool = False
    seed: int = 0
    # Values (kinds 2 and 5) are drawn with std input_std * v_std_ratio.
    v_std_ratio: float = 1.0

    def std(self, kind: int) -> float:
        """Standard deviation of the inputs of one kind (0-2 prefill Q/K/V,
        3-5 decode Q/K/V)."""
        return self.input_std * (self.v_std_ratio if kind in (2, 5) else 1.0)

    @property
    def batch(self) -> int:
        return len(self.prefill_lens)

    @property
    def elem_bytes(self) -> int:
        return 2 if self.dtype == "bf16" else 4

    def starts(self) -> Tuple[int, ...]:
        return self.start_steps or (0,) * self.batch

    def pool_rows(self) -> int:
        """Rows per layer: every request holds exactly prefill_len + W rows."""
        return sum(p + self.window for p in self.prefill_lens)

    def slot_bases(self) -> np.ndarray:
        """First logical row of each request in the (logical) pool."""
        sizes = np.array([p + self.window for p in self.prefill_lens], dtype=np.int64)
        return np.concatenate([[0], np.cumsum(sizes)[:-1]]).astype(np.int64)

    def slot_table(self) -> Optional[np.ndarray]:
        """Seeded shuffled permutation of pool rows (page-size-1 layout)."""
        if not self.paged:
            return None
        rng = np.random.default_rng([self.seed, self.wid, 99])
        return rng.permutation(self.pool_rows()).astype(np.int32)


def _ragged_prefill(seed: int, n: int, lo: int, hi: int) -> Tuple[int, ...]:
    rng = np.random.default_rng(seed)
    return tuple(int(p) for p in rng.integers(lo, hi + 1, n))


TINY = Workload(1, "tiny", layers=1, heads=2, head_dim=64, dtype="f32",
                prefill_lens=(32,), window=8, decode_steps=64, input_std=1.0)

SINGLE_PAGE = Workload(2, "single_page", layers=1, heads=10, head_dim=128, dtype="bf16",
                       prefill_lens=(TOKENS_PER_PAGE + 16,), window=WINDOW,
                       decode_steps=4096, input_std=1.0 / np.sqrt(128.0))

DOC16 = Workload(3, "doc16", layers=1, heads=10, head_dim=128, dtype="bf16",
                 prefill_lens=(16 * TOKENS_PER_PAGE + 64,) * 8, window=WINDOW,
                 decode_steps=16384, input_std=1.0 / np.sqrt(128.0))

DOC100 = Workload(4, "doc100", layers=1, heads=10, head_dim=128, dtype="bf16",
                  prefill_lens=(100 * TOKENS_PER_PAGE + 128,) * 4, window=WINDOW,
                  decode_steps=7000, input_std=1.0 / np.sqrt(128.0))

RAGGED = Workload(5, "ragged_mix", layers=12, heads=10, head_dim=128, dtype="bf16",
                  prefill_lens=_ragged_prefill(0, 64, TOKENS_PER_PAGE + 16,
                                               32 * TOKENS_PER_PAGE + 64),
                  window=WINDOW, decode_steps=2048, input_std=1.0 / np.sqrt(128.0),
                  start_steps=tuple(4 * r for r in range(64)), paged=True)

ALL = {w.name: w for w in (TINY, SINGLE_PAGE, DOC16, DOC100, RAGGED)}
