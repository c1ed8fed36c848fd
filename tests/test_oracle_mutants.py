"""Planted mistakes in the oracle must each fail at least one pin.

Each mutant replaces one oracle function (on the CPU, via monkeypatch) with a
plausible wrong variant: a sign, an index, an off-by-one window, a dropped
term.  If a mutant passed every pin, the pins would not be guarding that part
of the oracle.
"""

import numpy as np
import pytest

from oracle import rswa_oracle as O
import oracle_pins

_orig = {name: getattr(O, name) for name in dir(O) if not name.startswith("__")}
_orig_write = O.RingCache.write


def _rope_sign(x, pos, base=10000.0):
    return _orig["rope"](x, -np.asarray(pos, dtype=np.float64), base)


def _rope_shift(x, pos, base=10000.0):
    return _orig["rope"](x, np.asarray(pos, dtype=np.float64) + 1.0, base)


def _rope_interleaved(x, pos, base=10000.0):
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    perm = np.concatenate([np.arange(0, d, 2), np.arange(1, d, 2)])
    inv = np.argsort(perm)
    return _orig["rope"](x[..., perm], pos, base)[..., inv]


def _inv_freq_half(head_dim, base=10000.0):
    i = np.arange(head_dim // 2, dtype=np.float64)
    return np.power(float(base), -1.0 * i / head_dim)


def _write_rope_at_slot(self, k_new, v_new):
    slot = O.ring_slot(self.P, self.s, self.W)
    self.K[slot] = O.rope(np.asarray(k_new, dtype=np.float64), slot, self.base)
    self.V[slot] = np.asarray(v_new, dtype=np.float64)
    self.owner[slot] = self.s
    return slot


def _write_value_rotated(self, k_new, v_new):
    slot = _orig_write(self, k_new, v_new)
    self.V[slot] = O.rope(self.V[slot], O.position(self.P, self.s), self.base)
    return slot


def _mask_variant(extra_back, keep_prefill=True, include_current=True):
    def decode_mask(prefill_len, s, window):
        n = prefill_len + s + 1
        j = np.arange(n)
        first = prefill_len + max(0, s - window + 1 - extra_back)
        gen = j >= first
        if not include_current:
            gen &= j < n - 1
        if keep_prefill:
            return (j < prefill_len) | gen
        return j > n - 1 - window - extra_back
    return decode_mask


def _masked_attention_noscale(q, k, v, mask, scale):
    return _orig["masked_attention"](q, k, v, mask, 1.0)


def _masked_attention_axis0(q, k, v, mask, scale):
    q = np.asarray(q, dtype=np.float64)
    s = scale * (q @ np.asarray(k, dtype=np.float64).T)
    s = np.where(np.broadcast_to(mask, s.shape), s, -np.inf)
    p = np.exp(s - s.max(axis=1, keepdims=True))
    p = p / p.sum(axis=0, keepdims=True)
    return p @ np.asarray(v, dtype=np.float64)


_orig_attend = O.RingCache.attend


def _attend_swa_lo_shift(self, q, mode="rswa"):
    if mode != "swa":
        return _orig_attend(self, q, mode)
    n_valid = O.cache_len(self.P, self.s, self.W)
    q_hat = O.rope(np.asarray(q, dtype=np.float64), O.position(self.P, self.s), self.base)
    mask = np.ones((1, n_valid), dtype=bool)
    mask[0, : max(0, min(self.P, self.P + self.s + 2 - self.W))] = False
    return np.stack([O.masked_attention(q_hat[None, h], self.K[:n_valid, h], self.V[:n_valid, h],
                                        mask, self.scale)[0] for h in range(q_hat.shape[0])], axis=0)


MUTANTS = {
    "swa_window_one_too_wide": {"swa_decode_mask": lambda p, s, w: np.arange(p + s + 1) >= p + s - w},
    "swa_keeps_prefill": {"swa_decode_mask": lambda p, s, w: _orig["decode_mask"](p, s, w)},
    "swa_physical_window_start_shifted": {"RingCache.attend": _attend_swa_lo_shift},
    "rope_sign": {"rope": _rope_sign},
    "rope_shifted_position": {"rope": _rope_shift},
    "rope_interleaved_pairs": {"rope": _rope_interleaved},
    "rope_frequency_exponent": {"inv_freq": _inv_freq_half},
    "rope_key_at_slot_index": {"RingCache.write": _write_rope_at_slot},
    "value_rotated": {"RingCache.write": _write_value_rotated},
    "ring_pos_starts_at_one": {"ring_pos": lambda s, w: (s + 1) % w},
    "slot_without_prefill_offset": {"ring_slot": lambda p, s, w: s % w},
    "window_one_too_wide": {"decode_mask": _mask_variant(1)},
    "window_one_too_narrow": {"decode_mask": _mask_variant(-1)},
    "standard_swa_drops_prefill": {"decode_mask": _mask_variant(0, keep_prefill=False)},
    "current_token_excluded": {"decode_mask": _mask_variant(1, include_current=False)},
    "cache_len_before_write": {"cache_len": lambda p, s, w: p + min(s, w)},
    "no_softmax_scale": {"masked_attention": _masked_attention_noscale},
    "softmax_wrong_axis": {"masked_attention": _masked_attention_axis0},
    "causal_strict": {"causal_mask": lambda rows, n: np.arange(n)[None, :] < np.asarray(rows)[:, None]},
    "bidirectional_prefill": {"causal_mask": lambda rows, n: np.ones((len(rows), n), dtype=bool)},
    "kv_bytes_window_off_by_one": {
        "kv_read_bytes": lambda p, s, w, h, d, e: 2 * h * d * e * (p + min(s, w))},
    "prefill_flops_full_square": {"prefill_flops": lambda p, h, d: 4 * h * d * p * p // 2},
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, monkeypatch):
    for target, fn in MUTANTS[name].items():
        if target.startswith("RingCache."):
            monkeypatch.setattr(O.RingCache, target.split(".", 1)[1], fn)
        else:
            monkeypatch.setattr(O, target, fn)
    failed = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(O)
        except Exception as e:  # AssertionError, or the oracle refusing the input
            failed.append((pin.__name__, type(e).__name__))
    assert failed, f"mutant {name} passed every pin"
