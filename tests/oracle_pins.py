"""Pins for the R-SWA oracle: checks against things other than the oracle.

Each ``pin_*`` takes the oracle module and raises AssertionError when the
oracle disagrees with an independent route: hand-derived fixtures under
tests/golden/, closed forms, a deque simulation of the ring, brute-force
loops on tiny inputs, and torch's scaled_dot_product_attention in float64 on
the CPU.  test_oracle_pins.py runs them on the real oracle and
test_oracle_mutants.py checks that planted mistakes in the oracle fail at
least one of them.

Rotated inputs for the attention pins come from this file's own complex-number
rotation with hand-derived frequencies, not from the oracle's RoPE.
"""

from __future__ import annotations

import collections
import json
import math
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _rng(*key):
    return np.random.default_rng(list(key))


def complex_rope(x, pos, freqs):
    """Rotation as complex multiplication: (x1 + i x2) * exp(i pos f)."""
    x = np.asarray(x, dtype=np.float64)
    h = x.shape[-1] // 2
    z = x[..., :h] + 1j * x[..., h:]
    z = z * np.exp(1j * np.asarray(pos, dtype=np.float64)[..., None] * np.asarray(freqs))
    return np.concatenate([z.real, z.imag], axis=-1)


def _freqs(d):
    return np.array(_golden("rope_freqs.json")[f"D{d}"], dtype=np.float64)


def _sdpa(q, k, v, scale, mask=None, causal=False):
    """torch SDPA in float64 on the CPU.  q: [Tq, H, D], k/v: [Tk, H, D]."""
    import torch

    t = lambda a: torch.from_numpy(np.ascontiguousarray(np.asarray(a, np.float64).transpose(1, 0, 2)))[None]
    m = None if mask is None else torch.from_numpy(np.asarray(mask, dtype=bool))
    o = torch.nn.functional.scaled_dot_product_attention(
        t(q), t(k), t(v), attn_mask=m, is_causal=causal, scale=scale)
    return o[0].numpy().transpose(1, 0, 2)


# ---------------------------------------------------------------- RoPE pins

def pin_rope_identity_at_zero(O):
    x = _rng(1, 1).standard_normal((7, 3, 16))
    assert np.array_equal(O.rope(x, 0.0), x), "RoPE at position 0 must be the identity"


def pin_rope_frequencies(O):
    g = _golden("rope_freqs.json")
    for d in (2, 4, 8):
        f = O.inv_freq(d, g["base"])
        assert np.allclose(f, g[f"D{d}"], rtol=1e-15, atol=0), f"frequencies for D={d}: {f}"


def pin_rope_complex(O):
    """RoPE equals multiplication by exp(i p f) on (x[i], x[i+D/2]) pairs."""
    for d in (2, 4, 8):
        x = _rng(1, 2, d).standard_normal((9, 3, d))
        pos = np.array([0, 1, 2, 7, 100, 1000, 4095, 20000, 32767], dtype=np.float64)
        want = complex_rope(x, pos[:, None], _freqs(d))
        got = O.rope(x, pos[:, None], 10000.0)
        assert np.allclose(got, want, rtol=0, atol=1e-12), f"D={d} rotation differs"


def pin_rope_relative(O):
    """q.k after rotation depends only on the position difference."""
    rng = _rng(1, 3)
    q = rng.standard_normal(128)
    k = rng.standard_normal(128)
    for a, b, c in ((5, 3, 11), (100, 7, 2000), (0, 0, 31000), (32000, 1, 700)):
        d1 = O.rope(q, a) @ O.rope(k, b)
        d2 = O.rope(q, a + c) @ O.rope(k, b + c)
        assert abs(d1 - d2) < 1e-9 * (1 + abs(d1)), (a, b, c, d1, d2)


def pin_rope_norm(O):
    x = _rng(1, 4).standard_normal((50, 64))
    pos = np.arange(50) * 613.0
    y = O.rope(x, pos, 10000.0)
    h = 32
    assert np.allclose(x[:, :h] ** 2 + x[:, h:] ** 2, y[:, :h] ** 2 + y[:, h:] ** 2, atol=1e-12)


# ----------------------------------------------------------- attention pins

def pin_single_key_returns_value(O):
    rng = _rng(2, 1)
    q, k, v = (rng.standard_normal((1, 3, 8)) for _ in range(3))
    _, _, out = O.prefill(q, k, v)
    assert np.array_equal(out, v), "one visible key must return its value exactly"


def _brute_prefill(q_hat, k_hat, v, scale):
    """Pure-Python loops: softmax over keys j <= i, per head."""
    p_len, n_heads, d = q_hat.shape
    out = np.zeros_like(v)
    for h in range(n_heads):
        for i in range(p_len):
            logits = [scale * sum(q_hat[i, h, e] * k_hat[j, h, e] for e in range(d))
                      for j in range(i + 1)]
            mx = max(logits)
            w = [math.exp(x - mx) for x in logits]
            tot = sum(w)
            for e in range(d):
                out[i, h, e] = sum(w[j] * v[j, h, e] for j in range(i + 1)) / tot
    return out


def pin_prefill_bruteforce(O):
    rng = _rng(2, 2)
    p_len, n_heads, d = 6, 2, 4
    q, k, v = (rng.standard_normal((p_len, n_heads, d)) * 2 for _ in range(3))
    pos = np.arange(p_len, dtype=np.float64)[:, None]
    want = _brute_prefill(complex_rope(q, pos, _freqs(d)), complex_rope(k, pos, _freqs(d)), v,
                          1 / math.sqrt(d))
    k_hat, v_out, out = O.prefill(q, k, v, 10000.0)
    assert np.allclose(out, want, rtol=0, atol=1e-12), "prefill differs from brute force"
    assert np.allclose(k_hat, complex_rope(k, pos, _freqs(d)), atol=1e-12)
    assert np.array_equal(v_out, v)


def pin_prefill_vs_sdpa(O):
    rng = _rng(2, 3)
    p_len, n_heads, d = 41, 3, 8
    q, k, v = (rng.standard_normal((p_len, n_heads, d)) for _ in range(3))
    pos = np.arange(p_len, dtype=np.float64)[:, None]
    want = _sdpa(complex_rope(q, pos, _freqs(d)), complex_rope(k, pos, _freqs(d)), v,
                 1 / math.sqrt(d), causal=True)
    _, _, out = O.prefill(q, k, v, 10000.0)
    assert np.allclose(out, want, rtol=0, atol=1e-12), "prefill differs from SDPA(is_causal)"
    rows = np.array([0, 5, 40])
    _, _, out_rows = O.prefill(q, k, v, 10000.0, rows=rows)
    assert np.allclose(out_rows, want[rows], rtol=0, atol=1e-12), "row-sampled prefill differs"


# -------------------------------------------------------------- ring pins

def _deque_sim(p_len, window, steps):
    """Simulate the ring with a bounded FIFO of generated indices."""
    fifo = collections.deque(maxlen=window)
    owner = {}
    rows = []
    for s in range(steps):
        evicted = fifo[0] if len(fifo) == window else None
        if evicted is None:
            slot = p_len + len(fifo)
        else:
            slot = [r for r, o in owner.items() if o == evicted][0]
        fifo.append(s)
        owner[slot] = s
        rows.append(dict(slot=slot, evicted=evicted, visible=sorted(fifo),
                         cache_len=p_len + len(fifo)))
    return rows


def pin_ring_golden(O):
    g = _golden("ring_small.json")
    p_len, w = g["prefill_len"], g["window"]
    for i, s in enumerate(g["steps"]):
        assert O.ring_pos(s, w) == g["ring_pos"][i]
        assert O.ring_slot(p_len, s, w) == g["slot"][i]
        assert O.position(p_len, s) == g["position"][i]
        assert O.cache_len(p_len, s, w) == g["cache_len"][i]
        assert O.evicted_index(s, w) == g["evicted"][i]
        m = O.decode_mask(p_len, s, w)
        gen = [j - p_len for j in np.flatnonzero(m) if j >= p_len]
        assert gen == g["visible_generated"][i], (s, gen)
        assert m[:p_len].all()


def pin_ring_vs_deque(O):
    for p_len, w, n in ((0, 1, 10), (3, 1, 9), (5, 3, 20), (17, 8, 70), (272, 128, 400)):
        sim = _deque_sim(p_len, w, n)
        for s, row in enumerate(sim):
            assert O.ring_slot(p_len, s, w) == row["slot"], (p_len, w, s)
            assert O.cache_len(p_len, s, w) == row["cache_len"], (p_len, w, s)
            assert O.evicted_index(s, w) == row["evicted"], (p_len, w, s)
            m = O.decode_mask(p_len, s, w)
            assert len(m) == p_len + s + 1
            assert list(np.flatnonzero(m[p_len:])) == row["visible"], (p_len, w, s)
            assert m[:p_len].all()
        # physical cache: which generated index each ring row holds
        d = 4
        rc = O.RingCache(p_len, w, 1, d)
        rc.load_prefill(np.zeros((p_len, 1, d)), np.zeros((p_len, 1, d)))
        for s, row in enumerate(sim):
            rc.step(np.zeros((1, d)), np.zeros((1, d)), np.zeros((1, d)))
            held = sorted(int(o) for o in rc.owner[p_len:] if o >= 0)
            assert held == row["visible"], (p_len, w, s, held)


def pin_cache_len_constant(O):
    """Once warm, the cache holds prefill_len + W entries however long decode runs."""
    for p_len, w in ((0, 4), (272, 128), (25728, 128)):
        for s in list(range(w - 1, w + 300)) + [10_000, 100_000]:
            assert O.cache_len(p_len, s, w) == p_len + w
        for s in range(0, w - 1):
            assert O.cache_len(p_len, s, w) < p_len + w


# ------------------------------------------------------------ decode pins

def _run_decode(O, p_len, w, n_steps, n_heads, d, seed, scale_in=1.0):
    rng = _rng(3, seed)
    pq, pk, pv = (rng.standard_normal((p_len, n_heads, d)) * scale_in for _ in range(3))
    dq, dk, dv = (rng.standard_normal((n_steps, n_heads, d)) * scale_in for _ in range(3))
    return pq, pk, pv, dq, dk, dv


def pin_decode_uniform_query_counts(O):
    """With q = 0 attention is the plain mean of the visible values.

    Values are one-hot by logical position, so the output times the number of
    visible positions is exactly the indicator of the visible set.  The set is
    the whole prefill plus the generated indices the FIFO simulation holds.
    """
    p_len, w, n, d = 9, 4, 30, 64
    eye = np.eye(d)
    k_all = _rng(3, 9).standard_normal((p_len + n, 1, d))
    v_all = eye[: p_len + n][:, None, :]
    sim = _deque_sim(p_len, w, n)
    rc = O.RingCache(p_len, w, 1, d)
    rc.load_prefill(k_all[:p_len], v_all[:p_len])
    for s in range(n):
        vis = list(range(p_len)) + [p_len + j for j in sim[s]["visible"]]
        want = np.zeros(d)
        want[vis] = 1.0 / len(vis)
        got = O.decode_logical(np.zeros((1, d)), k_all[: p_len + s + 1], v_all[: p_len + s + 1],
                               p_len, s, w)[0]
        assert np.allclose(got, want, atol=1e-15), ("logical", s)
        got_p = rc.step(np.zeros((1, d)), k_all[p_len + s], v_all[p_len + s])[0]
        assert np.allclose(got_p, want, atol=1e-15), ("physical", s)


def pin_decode_warmup_is_full_causal(O):
    """While s < W nothing is evicted: decode = causal attention over everything."""
    p_len, w, n, h, d = 13, 16, 16, 2, 8
    pq, pk, pv, dq, dk, dv = _run_decode(O, p_len, w, n, h, d, 1)
    q = np.concatenate([pq, dq])
    k = np.concatenate([pk, dk])
    v = np.concatenate([pv, dv])
    pos = np.arange(p_len + n, dtype=np.float64)[:, None]
    want = _sdpa(complex_rope(q, pos, _freqs(d)), complex_rope(k, pos, _freqs(d)), v,
                 1 / math.sqrt(d), causal=True)
    rc = O.RingCache(p_len, w, h, d)
    rc.load_prefill(pk, pv)
    for s in range(n):
        got_l = O.decode_logical(dq[s], k[: p_len + s + 1], v[: p_len + s + 1], p_len, s, w)
        got_p = rc.step(dq[s], dk[s], dv[s])
        assert np.allclose(got_l, want[p_len + s], atol=1e-12), ("logical", s)
        assert np.allclose(got_p, want[p_len + s], atol=1e-12), ("physical", s)


def pin_decode_no_prefill_is_textbook_swa(O):
    """P = 0: query i sees keys i-W < j <= i (sliding-window causal attention)."""
    w, n, h, d = 5, 23, 2, 8
    _, _, _, dq, dk, dv = _run_decode(O, 0, w, n, h, d, 2)
    pos = np.arange(n, dtype=np.float64)[:, None]
    i = np.arange(n)[:, None]
    j = np.arange(n)[None, :]
    band = (j <= i) & (i - j < w)
    want = _sdpa(complex_rope(dq, pos, _freqs(d)), complex_rope(dk, pos, _freqs(d)), dv,
                 1 / math.sqrt(d), mask=band)
    rc = O.RingCache(0, w, h, d)
    rc.load_prefill(np.zeros((0, h, d)), np.zeros((0, h, d)))
    for s in range(n):
        got_l = O.decode_logical(dq[s], dk[: s + 1], dv[: s + 1], 0, s, w)
        got_p = rc.step(dq[s], dk[s], dv[s])
        assert np.allclose(got_l, want[s], atol=1e-12), ("logical", s)
        assert np.allclose(got_p, want[s], atol=1e-12), ("physical", s)


def pin_decode_huge_window_is_full_causal(O):
    p_len, n, h, d = 6, 30, 1, 8
    w = n + 5
    pq, pk, pv, dq, dk, dv = _run_decode(O, p_len, w, n, h, d, 3)
    q = np.concatenate([pq, dq])
    k = np.concatenate([pk, dk])
    v = np.concatenate([pv, dv])
    pos = np.arange(p_len + n, dtype=np.float64)[:, None]
    want = _sdpa(complex_rope(q, pos, _freqs(d)), complex_rope(k, pos, _freqs(d)), v,
                 1 / math.sqrt(d), causal=True)
    for s in range(n):
        got = O.decode_logical(dq[s], k[: p_len + s + 1], v[: p_len + s + 1], p_len, s, w)
        assert np.allclose(got, want[p_len + s], atol=1e-12), s


def pin_physical_equals_logical(O):
    """The in-place ring (any slot order) equals the explicit-mask form."""
    for p_len, w, n in ((7, 3, 25), (0, 2, 9), (20, 8, 40)):
        h, d = 2, 16
        pq, pk, pv, dq, dk, dv = _run_decode(O, p_len, w, n, h, d, 4 + w)
        k = np.concatenate([pk, dk])
        v = np.concatenate([pv, dv])
        rc = O.RingCache(p_len, w, h, d)
        rc.load_prefill(pk, pv)
        for s in range(n):
            got_p = rc.step(dq[s], dk[s], dv[s])
            got_l = O.decode_logical(dq[s], k[: p_len + s + 1], v[: p_len + s + 1], p_len, s, w)
            assert np.allclose(got_p, got_l, rtol=0, atol=1e-12), (p_len, w, s)


def pin_planted_keys(O):
    """A key planted along the query decides the output only while visible."""
    p_len, w, n, h, d = 10, 4, 12, 1, 16
    rng = _rng(3, 77)
    pk, pv = rng.standard_normal((p_len, h, d)), rng.standard_normal((p_len, h, d))
    dk, dv = rng.standard_normal((n, h, d)) * 0.1, rng.standard_normal((n, h, d))
    k = np.concatenate([pk, dk])
    v = np.concatenate([pv, dv])
    s = n - 1                      # generated index s - W = 7 was just evicted
    gone = s - w
    pos = np.arange(p_len + n)
    # direction q whose rotation at P+s matches the rotated planted key
    for target, expect_hit in ((p_len + gone, False), (3, True), (p_len + s - 1, True)):
        kk = k.copy()
        kk[target, 0] = rng.standard_normal(d)
        k_hat_t = O.rope(kk[target], pos[target])
        q_hat = 60.0 * k_hat_t / np.linalg.norm(k_hat_t) ** 2 * np.sqrt(d)
        # undo the query rotation at position P+s: rotate by the negative position
        q = O.rope(q_hat, -(p_len + s))
        out = O.decode_logical(q, kk[: p_len + s + 1], v[: p_len + s + 1], p_len, s, w)[0]
        dist = np.abs(out - v[target, 0]).max()
        if expect_hit:
            assert dist < 1e-6, (target, dist)
        else:
            assert dist > 0.1, (target, dist)


# ------------------------------------------- standard-window baseline (SWA)

def pin_swa_is_textbook_band(O):
    """The standard-window baseline: query at position i sees keys
    i - W < j <= i over prefill and generated tokens alike; checked for the
    logical and the physical form against banded SDPA in fp64."""
    for p_len, w, n in ((9, 4, 20), (0, 3, 11), (5, 12, 14), (30, 7, 9)):
        h, d = 2, 8
        pq, pk, pv, dq, dk, dv = _run_decode(O, p_len, w, n, h, d, 40 + p_len + w)
        q = np.concatenate([pq, dq])
        k = np.concatenate([pk, dk])
        v = np.concatenate([pv, dv])
        tot = p_len + n
        pos = np.arange(tot, dtype=np.float64)[:, None]
        i = np.arange(tot)[:, None]
        j = np.arange(tot)[None, :]
        band = (j <= i) & (i - j < w)
        want = _sdpa(complex_rope(q, pos, _freqs(d)), complex_rope(k, pos, _freqs(d)), v,
                     1 / math.sqrt(d), mask=band)
        rc = O.RingCache(p_len, w, h, d)
        rc.load_prefill(pk, pv)
        for st in range(n):
            got_l = O.decode_logical(dq[st], k[: p_len + st + 1], v[: p_len + st + 1], p_len, st, w,
                                     mode="swa")
            got_p = rc.step(dq[st], dk[st], dv[st], mode="swa")
            assert np.allclose(got_l, want[p_len + st], atol=1e-12), ("logical", p_len, w, st)
            assert np.allclose(got_p, want[p_len + st], atol=1e-12), ("physical", p_len, w, st)


def pin_swa_visible_set(O):
    """q = 0 with one-hot values: the output is the indicator of the visible
    positions divided by their number; the baseline sees exactly the last
    min(W, P + s + 1) positions, a subset of what R-SWA sees."""
    p_len, w, n, d = 11, 4, 20, 64
    eye = np.eye(d)
    k_all = _rng(5, 9).standard_normal((p_len + n, 1, d))
    v_all = eye[: p_len + n][:, None, :]
    rc = O.RingCache(p_len, w, 1, d)
    rc.load_prefill(k_all[:p_len], v_all[:p_len])
    for st in range(n):
        last = p_len + st
        vis = list(range(max(0, last - w + 1), last + 1))
        want = np.zeros(d)
        want[vis] = 1.0 / len(vis)
        got = O.decode_logical(np.zeros((1, d)), k_all[: last + 1], v_all[: last + 1], p_len, st, w,
                               mode="swa")[0]
        assert np.allclose(got, want, atol=1e-15), ("logical", st)
        got_p = rc.step(np.zeros((1, d)), k_all[last], v_all[last], mode="swa")[0]
        assert np.allclose(got_p, want, atol=1e-15), ("physical", st)
        assert set(np.flatnonzero(O.swa_decode_mask(p_len, st, w))) <= \
            set(np.flatnonzero(O.decode_mask(p_len, st, w)))


# ------------------------------------------------------------- work counts

def pin_work_counts(O):
    for p_len, w, h, d, eb in ((5, 3, 2, 8, 2), (272, 128, 10, 128, 2), (32, 8, 2, 64, 4)):
        for s in (0, 1, w - 1, w, 3 * w + 1):
            n_vis = int(O.decode_mask(p_len, s, w).sum())
            assert n_vis == len(_deque_sim(p_len, w, s + 1)[s]["visible"]) + p_len
            assert O.kv_read_bytes(p_len, s, w, h, d, eb) == 2 * h * d * eb * n_vis
        pairs = sum(i + 1 for i in range(p_len))
        assert O.prefill_flops(p_len, h, d) == 2 * 2 * h * d * pairs


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
