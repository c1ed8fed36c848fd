"""The n-gram ban oracle against its pins, and planted mistakes in it
(monkeypatched on the CPU) each failing at least one pin."""

import pytest

from oracle import ngram_oracle as N
import ngram_pins

_orig = N.banned_tokens


@pytest.mark.parametrize("pin", ngram_pins.ALL, ids=lambda p: p.__name__)
def test_pin(pin):
    pin(N)


def _variant(w0_shift=0, last_excluded=False, prefix_len_delta=0, ignore_window=False,
             start_before_window=0):
    def banned_tokens(seq, n, window):
        seq = [int(t) for t in seq]
        length = len(seq)
        if n < 1 or length < n or window < n:
            return set()
        w0 = 0 if ignore_window else max(0, length - window + w0_shift - start_before_window)
        k = n - 1 + prefix_len_delta
        prefix = seq[length - k:] if k > 0 else []
        hi = length - n + (0 if last_excluded else 1)
        out = set()
        for i in range(w0, hi):
            if seq[i:i + k] == prefix and i + n - 1 < length:
                out.add(seq[i + n - 1])
        return out
    return banned_tokens


MUTANTS = {
    "window_start_plus_one": _variant(w0_shift=1),
    "window_start_minus_one": _variant(start_before_window=1),
    "last_ngram_excluded": _variant(last_excluded=True),
    "prefix_one_short": _variant(prefix_len_delta=-1),
    "prefix_one_long": _variant(prefix_len_delta=1),
    "window_ignored": _variant(ignore_window=True),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, monkeypatch):
    monkeypatch.setattr(N, "banned_tokens", MUTANTS[name])
    failed = []
    for pin in ngram_pins.ALL:
        try:
            pin(N)
        except AssertionError:
            failed.append(pin.__name__)
    assert failed, f"mutant {name} passed every pin"
