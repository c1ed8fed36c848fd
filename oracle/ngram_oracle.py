"""Oracle for the windowed no-repeat n-gram logits processor: plain Python.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU
baseline leg of the benchmark may import or call this module.  The product
path never does, and this module imports nothing from it.

Source: [T5 §2.3] page "开源5天Star破万之后：百度Unlimited-OCR的爆火路径复盘"
(www.gtnt.cn/news/146005), section 2.3 "反循环采样" (anti-loop sampling).
Long decoding can fall into an n-gram loop; the model's processor checks for
repeats only inside a sliding window rather than over the whole sequence,
and sets to -inf the score of every token that would reproduce an n-gram of
ngram_size tokens.  Its defaults are ngram_size = 35 and window = 128; the
vocabulary has 129,280 tokens (section 2.4).

Reading taken (the page prints no code): for a token sequence x_0 .. x_{L-1}
the window is its last min(window, L) tokens, x_{w0} .. x_{L-1} with
w0 = max(0, L - window).  Every n-gram lying wholly inside the window,
x_i .. x_{i+n-1} with w0 <= i <= L - n, whose first n - 1 tokens equal the
sequence's last n - 1 tokens x_{L-n+1} .. x_{L-1}, bans its last token
x_{i+n-1}: choosing it next would repeat that n-gram.  When L < n or
window < n no n-gram fits and nothing is banned.  For n = 1 the prefix is
empty and every token in the window is banned.  Tokens outside
[0, vocab) are never banned (no logit exists for them).
"""

from __future__ import annotations

import numpy as np


def banned_tokens(seq, n: int, window: int):
    """Set of tokens banned after the sequence seq [T5 §2.3]."""
    seq = [int(t) for t in seq]
    length = len(seq)
    if n < 1 or length < n or window < n:
        return set()
    w0 = max(0, length - window)
    prefix = seq[length - n + 1:]            # last n - 1 tokens (empty for n = 1)
    banned = set()
    for i in range(w0, length - n + 1):      # n-grams wholly inside the window
        if seq[i:i + n - 1] == prefix:
            banned.add(seq[i + n - 1])
    return banned


def apply(logits, seqs, n: int, window: int):
    """Copy of logits [requests][vocab] with -inf at each request's banned
    tokens that lie in [0, vocab) [T5 §2.3]."""
    out = np.array(logits, copy=True)
    vocab = out.shape[1]
    for r, seq in enumerate(seqs):
        for t in banned_tokens(seq, n, window):
            if 0 <= t < vocab:
                out[r, t] = -np.inf
    return out
