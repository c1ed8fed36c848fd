"""Pins for the n-gram ban oracle: checks against routes other than the
oracle's own prefix scan.

* hand-worked cases in tests/golden/ngram_small.json (page section 2.3
  reading, each with its derivation);
* a full n-gram search: token t is banned exactly when the n-gram
  (last n - 1 tokens, t) occurs as a contiguous run wholly inside the window,
  checked for every t of a tiny vocabulary;
* with the window covering the whole sequence, a dictionary of all n-grams
  (prefix tuple -> set of next tokens) looked up at the last n - 1 tokens;
* the ban set only grows with the window, and tokens before the window do
  not matter;
* apply() changes exactly the banned in-range logits, to -inf.
"""

from __future__ import annotations

import json
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rng_seqs(seed, count, vocab, max_len):
    """Short sequences over a tiny vocabulary, with loops planted so that
    bans are common."""
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(count):
        length = int(rng.integers(0, max_len + 1))
        period = int(rng.integers(1, 6))
        base = rng.integers(0, vocab, period)
        seq = [int(base[i % period]) for i in range(length)]
        for i in range(length):                   # break the loop here and there
            if rng.random() < 0.15:
                seq[i] = int(rng.integers(0, vocab))
        out.append(seq)
    return out


def pin_golden(N):
    doc = json.load(open(os.path.join(GOLDEN, "ngram_small.json")))
    for c in doc["cases"]:
        got = sorted(N.banned_tokens(c["seq"], c["n"], c["window"]))
        assert got == c["banned"], (c, got)


def pin_full_ngram_search(N):
    vocab = 5
    for seq in _rng_seqs(1, 300, vocab, 24):
        for n in (1, 2, 3, 4):
            for window in (1, 3, 6, 11, 40):
                banned = N.banned_tokens(seq, n, window)
                win = seq[max(0, len(seq) - window):]
                for t in range(vocab):
                    cand = seq[len(seq) - (n - 1):] + [t] if n > 1 else [t]
                    occurs = len(seq) >= n and any(win[i:i + n] == cand
                                                   for i in range(len(win) - n + 1))
                    assert (t in banned) == occurs, (seq, n, window, t)


def pin_whole_sequence_dictionary(N):
    for seq in _rng_seqs(2, 200, 7, 30):
        for n in (1, 2, 3, 5):
            table = {}
            for i in range(len(seq) - n + 1):
                table.setdefault(tuple(seq[i:i + n - 1]), set()).add(seq[i + n - 1])
            want = table.get(tuple(seq[len(seq) - n + 1:]), set()) if len(seq) >= n else set()
            assert N.banned_tokens(seq, n, len(seq) + 3) == want, (seq, n)


def pin_window_monotone_and_local(N):
    for seq in _rng_seqs(3, 150, 4, 28):
        for n in (2, 3):
            prev = set()
            for window in range(0, len(seq) + 2):
                cur = N.banned_tokens(seq, n, window)
                assert prev <= cur, (seq, n, window)
                prev = cur
            window = 6
            if len(seq) > window:
                assert N.banned_tokens(seq, n, window) == N.banned_tokens(seq[-window:], n, window)
                assert N.banned_tokens([3, 3, 3] + seq, n, window) == N.banned_tokens(seq, n, window)


def pin_apply(N):
    rng = np.random.default_rng(4)
    seqs = [[1, 2, 1, 2, 1], [0, 0, 0], [9, 9, 2, 9, 9], []]
    logits = rng.standard_normal((4, 6)).astype(np.float32)
    out = N.apply(logits, seqs, 2, 8)
    # request 0: prefix (1) -> 2; request 1: prefix (0) -> 0;
    # request 2: prefix (9) -> 9 and 2; token 9 is outside the vocabulary of 6
    want = logits.copy()
    want[0, 2] = -np.inf
    want[1, 0] = -np.inf
    want[2, 2] = -np.inf
    assert np.array_equal(out, want)
    assert out.dtype == logits.dtype


ALL = [pin_golden, pin_full_ngram_search, pin_whole_sequence_dictionary,
       pin_window_monotone_and_local, pin_apply]
