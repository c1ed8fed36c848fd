"""Oracle for Reference Sliding Window Attention (R-SWA): plain, slow, fp64.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU
baseline leg of the benchmark may import or call this module.  The product
path (the HIP library and its Python binding) never does, and this module
imports nothing from it.

Sources, cited by page title and section:

* [T5 §2.1] page "开源5天Star破万之后：百度Unlimited-OCR的爆火路径复盘"
  (www.gtnt.cn/news/146005), section 2.1 "环形滑窗注意力" (ring
  sliding-window attention).  It fixes the method: the prefill segment keeps
  complete attention and loses no token; decode keys/values are appended until
  the cache holds prefill_len + W entries; after that every new token
  overwrites, in place, the ring slot that follows the prefill, at
  slot = prefill_len + ring_pos with ring_pos advancing by one modulo W, and
  attention then runs over the whole cache.  The cache therefore never grows
  beyond prefill_len + W.  The same section gives W = 128
  (sliding_window_size), max_position_embeddings = 32768, and about 256
  image tokens per 1024x1024 page.  It contrasts the method with a standard
  sliding window, which would also cut the prefill keys/values.
* [T5 §3] same page, section 三 (ecosystem and engines): the eager transformers
  path computes prefill attention with a full-matrix softmax.
* [T4] page "Kimi K3 và Unlimited OCR chiếm lĩnh top 2 toàn cầu..." (aihot.vn,
  QbitAI repost), R-SWA paragraph: attention keeps the original document in
  focus and holds only the most recently generated content as working memory.

Readings taken where the pages are silent (each stated where it is used):

* RoPE is not on the pages.  Keys and queries are rotated with the
  rotate-half (Llama / GPT-NeoX) convention over the whole head dimension,
  frequencies base^(-2i/D), at the token's absolute position: prefill token j
  at position j, decode step s at position prefill_len + s.  Keys are stored
  already rotated; values are never rotated.
* ring_pos starts at 0 for the first decode step, so during warm-up the slot
  formula coincides with plain appending and eviction is first-in first-out.
* The key/value of the current token is written before attention, so the
  window of generated keys includes the current token: W generated keys once
  warm, min(s + 1, W) at step s during warm-up.
* Prefill "full attention" is causal (a decoder), not bidirectional.
* Softmax scale 1/sqrt(D) unless given; key heads equal query heads.

Every function works in float64 on numpy arrays.  Inputs are whatever the
caller passes (already rounded to the run dtype); nothing is rounded here.
Shapes use T tokens, H heads, D head dimension.
"""

from __future__ import annotations

import numpy as np

__all__ = [
    "inv_freq",
    "rope",
    "masked_attention",
    "causal_mask",
    "prefill",
    "ring_pos",
    "ring_slot",
    "position",
    "cache_len",
    "evicted_index",
    "decode_mask",
    "decode_logical",
    "RingCache",
    "kv_read_bytes",
    "prefill_flops",
]


# --------------------------------------------------------------------------
# Rotary position embedding (reading: not on the pages, see module docstring)
# --------------------------------------------------------------------------

def inv_freq(head_dim: int, base: float = 10000.0) -> np.ndarray:
    """Per-pair rotation frequencies f_i = base^(-2i/D), i = 0 .. D/2-1."""
    if head_dim % 2:
        raise ValueError("head_dim must be even")
    i = np.arange(head_dim // 2, dtype=np.float64)
    return np.power(float(base), -2.0 * i / head_dim)


def rope(x, pos, base: float = 10000.0) -> np.ndarray:
    """Rotate-half RoPE of x[..., D] at positions pos.

    pos must broadcast against x.shape[:-1] (pass pos[:, None] for x of shape
    [T, H, D]).  For i < D/2, with a = pos * f_i:
        out[i]       = x[i] cos a - x[i + D/2] sin a
        out[i + D/2] = x[i + D/2] cos a + x[i] sin a
    """
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    h = d // 2
    ang = np.asarray(pos, dtype=np.float64)[..., None] * inv_freq(d, base)
    c = np.cos(ang)
    s = np.sin(ang)
    x1 = x[..., :h]
    x2 = x[..., h:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


# --------------------------------------------------------------------------
# Attention by definition: softmax over an explicit boolean mask
# --------------------------------------------------------------------------

def masked_attention(q, k, v, mask, scale: float) -> np.ndarray:
    """o_i = sum_j softmax_j(scale * q_i . k_j restricted to mask[i]) v_j.

    q: [Tq, D]; k, v: [Tk, D]; mask: [Tq, Tk] bool (True = key visible).
    The row maximum is subtracted before exponentiation (exact in real
    arithmetic).  Every row must see at least one key.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    mask = np.broadcast_to(np.asarray(mask, dtype=bool), (q.shape[0], k.shape[0]))
    if not mask.any(axis=1).all():
        raise ValueError("a query row sees no key")
    s = scale * (q @ k.T)
    s = np.where(mask, s, -np.inf)
    m = s.max(axis=1, keepdims=True)
    p = np.exp(s - m)
    p = p / p.sum(axis=1, keepdims=True)
    return p @ v


def causal_mask(rows, n_keys: int) -> np.ndarray:
    """Causal visibility: query at position i sees keys j <= i."""
    rows = np.asarray(rows)
    return np.arange(n_keys)[None, :] <= rows[:, None]


def _default_scale(d: int, scale):
    return 1.0 / np.sqrt(d) if scale is None or scale <= 0 else float(scale)


# --------------------------------------------------------------------------
# Prefill: complete causal attention over the prefill, nothing evicted
# [T5 §2.1], full-matrix softmax as the eager path does it [T5 §3]
# --------------------------------------------------------------------------

def prefill(q, k, v, base: float = 10000.0, scale=None, rows=None):
    """Causal prefill of one request.

    q, k, v: [P, H, D] (unrotated).  Returns (k_hat, v, out):
      k_hat[j] = RoPE(k[j], j)   -- what the cache holds for slot j
      out[r]   = causal attention output of query row rows[r] (all rows if
                 rows is None), with q rotated at its own position.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    p_len, n_heads, d = q.shape
    sc = _default_scale(d, scale)
    pos = np.arange(p_len)
    k_hat = rope(k, pos[:, None], base)
    rows = pos if rows is None else np.asarray(rows, dtype=np.int64)
    q_hat = rope(q[rows], rows[:, None], base)
    mask = causal_mask(rows, p_len)
    out = np.stack(
        [masked_attention(q_hat[:, h], k_hat[:, h], v[:, h], mask, sc)
         for h in range(n_heads)],
        axis=1,
    )
    return k_hat, v, out


# --------------------------------------------------------------------------
# Ring bookkeeping (integers) [T5 §2.1]
# Step s is the s-th decode token of a request, s = 0, 1, 2, ...
# --------------------------------------------------------------------------

def ring_pos(s: int, window: int) -> int:
    """ring_pos used by decode step s: starts at 0, advances by one mod W."""
    return s % window


def ring_slot(prefill_len: int, s: int, window: int) -> int:
    """Cache slot written by step s: the ring slot after the prefill."""
    return prefill_len + ring_pos(s, window)


def position(prefill_len: int, s: int) -> int:
    """Absolute position of decode step s (prefill occupies 0 .. P-1)."""
    return prefill_len + s


def cache_len(prefill_len: int, s: int, window: int) -> int:
    """Number of valid cache entries once step s has written its key/value.

    Grows by one per step during warm-up, then stays at prefill_len + W.
    """
    return prefill_len + min(s + 1, window)


def evicted_index(s: int, window: int):
    """Generated-token index whose slot step s overwrites (None in warm-up)."""
    return s - window if s >= window else None


# --------------------------------------------------------------------------
# Decode, logical form: explicit mask over logical positions 0 .. P+s
# --------------------------------------------------------------------------

def decode_mask(prefill_len: int, s: int, window: int) -> np.ndarray:
    """Visibility of logical positions 0 .. P+s for the query of step s.

    Every prefill position is visible; of the generated positions
    P .. P+s only the newest min(s + 1, W) are (the current one included).
    """
    n = prefill_len + s + 1
    j = np.arange(n)
    first_gen = prefill_len + max(0, s - window + 1)
    return (j < prefill_len) | (j >= first_gen)


def swa_decode_mask(prefill_len: int, s: int, window: int) -> np.ndarray:
    """Baseline: a standard sliding window [T5 §2.1, the contrast it draws].

    The query of step s sees the newest W logical positions of 0 .. P+s,
    prefill and generated alike (the current one included), so once the
    window has moved past the prefill its keys are gone.  Reading: the
    window is applied at decode; prefill attention stays causal.
    """
    n = prefill_len + s + 1
    return np.arange(n) >= n - window


def decode_logical(q_s, k_hist, v_hist, prefill_len: int, s: int, window: int,
                   base: float = 10000.0, scale=None, mode: str = "rswa") -> np.ndarray:
    """Output of decode step s from the full history, masked explicitly.

    q_s: [H, D] unrotated query of step s.
    k_hist, v_hist: [P+s+1, H, D] unrotated keys / values of logical
    positions 0 .. P+s (prefill tokens, then generated tokens 0 .. s).
    mode "rswa" uses decode_mask, "swa" the standard-window baseline.
    Returns [H, D].
    """
    k_hist = np.asarray(k_hist, dtype=np.float64)
    v_hist = np.asarray(v_hist, dtype=np.float64)
    n, n_heads, d = k_hist.shape
    if n != prefill_len + s + 1:
        raise ValueError("history length must be P + s + 1")
    sc = _default_scale(d, scale)
    pos = np.arange(n)
    k_hat = rope(k_hist, pos[:, None], base)
    q_hat = rope(np.asarray(q_s, dtype=np.float64), position(prefill_len, s), base)
    mask_fn = {"rswa": decode_mask, "swa": swa_decode_mask}[mode]
    mask = mask_fn(prefill_len, s, window)[None, :]
    return np.stack(
        [masked_attention(q_hat[None, h], k_hat[:, h], v_hist[:, h], mask, sc)[0]
         for h in range(n_heads)],
        axis=0,
    )


# --------------------------------------------------------------------------
# Decode, physical form: a cache of P + W rows with an in-place ring
# --------------------------------------------------------------------------

class RingCache:
    """One request's R-SWA cache, simulated row by row.

    Rows 0 .. P-1 hold the rotated prefill keys and values and never change.
    Rows P .. P+W-1 are the ring.  Unwritten rows hold NaN so that reading
    one poisons the result.
    """

    def __init__(self, prefill_len: int, window: int, n_heads: int, head_dim: int,
                 base: float = 10000.0, scale=None):
        if window < 1 or prefill_len < 0:
            raise ValueError("need W >= 1 and P >= 0")
        self.P = int(prefill_len)
        self.W = int(window)
        self.base = float(base)
        self.scale = _default_scale(head_dim, scale)
        rows = self.P + self.W
        self.K = np.full((rows, n_heads, head_dim), np.nan)
        self.V = np.full((rows, n_heads, head_dim), np.nan)
        self.owner = np.full(rows, -1, dtype=np.int64)  # generated index per ring row
        self.s = 0

    def load_prefill(self, k, v):
        """Store the prefill keys (rotated at positions 0..P-1) and values."""
        k = np.asarray(k, dtype=np.float64)
        if k.shape[0] != self.P:
            raise ValueError("prefill length mismatch")
        self.K[: self.P] = rope(k, np.arange(self.P)[:, None], self.base)
        self.V[: self.P] = np.asarray(v, dtype=np.float64)
        self.s = 0

    def write(self, k_new, v_new) -> int:
        """Write the current step's key (rotated at its position) and value."""
        slot = ring_slot(self.P, self.s, self.W)
        pos = position(self.P, self.s)
        self.K[slot] = rope(np.asarray(k_new, dtype=np.float64), pos, self.base)
        self.V[slot] = np.asarray(v_new, dtype=np.float64)
        self.owner[slot] = self.s
        return slot

    def attend(self, q, mode: str = "rswa") -> np.ndarray:
        """Attention of the current step's query over the valid cache rows:
        all of them (R-SWA), or for the standard-window baseline only the
        ring and the prefill rows at positions >= P + s + 1 - W."""
        n_valid = cache_len(self.P, self.s, self.W)
        q_hat = rope(np.asarray(q, dtype=np.float64), position(self.P, self.s), self.base)
        mask = np.ones((1, n_valid), dtype=bool)
        if mode == "swa":
            mask[0, : max(0, min(self.P, self.P + self.s + 1 - self.W))] = False
        return np.stack(
            [masked_attention(q_hat[None, h], self.K[:n_valid, h], self.V[:n_valid, h],
                              mask, self.scale)[0]
             for h in range(q_hat.shape[0])],
            axis=0,
        )

    def step(self, q, k_new, v_new, mode: str = "rswa") -> np.ndarray:
        """One decode step: write, attend, advance.  Returns [H, D]."""
        self.write(k_new, v_new)
        out = self.attend(q, mode)
        self.s += 1
        return out


# --------------------------------------------------------------------------
# Work counts used to express throughput (algorithmic, not implementation)
# --------------------------------------------------------------------------

def kv_read_bytes(prefill_len: int, s: int, window: int, n_heads: int, head_dim: int,
                  elem_bytes: int) -> int:
    """Key + value bytes decode step s must read for one request and layer."""
    return 2 * n_heads * head_dim * elem_bytes * cache_len(prefill_len, s, window)


def prefill_flops(prefill_len: int, n_heads: int, head_dim: int) -> int:
    """Multiply-add work of causal prefill attention, counted as 2 flops each.

    Per head, q.k and p.v each take D multiply-adds per visible pair, and a
    causal prefill of P tokens has P(P+1)/2 visible pairs.
    """
    return 4 * n_heads * head_dim * prefill_len * (prefill_len + 1) // 2
