"""Layout invariants of the bf16 prefill kernel's LDS tiles (host-side model
of the address arithmetic in csrc/rswa_prefill_mfma.hip, no GPU needed).

A K or V tile is 64 key rows of D bf16, unpadded; 16-byte chunk c of row r
sits at position c ^ swz(r).  The checks: every row's chunks land on
distinct positions (the loads that fill a tile write each chunk exactly
once), and the two read patterns of the kernel touch distinct LDS banks
(64 banks of 4 bytes) within each group of lanes that the hardware serves
together, so neither read is slowed by bank conflicts."""

import itertools

import pytest


def swz(d, r):
    if d == 128:
        return 4 * (r & 3) + ((r >> 2) & 3)
    return 4 * ((r >> 1) & 1) + ((r >> 2) & 3)


def byte_of(d, row, chunk):
    """LDS byte offset of chunk `chunk` of key row `row` inside a tile."""
    return row * 2 * d + (chunk ^ swz(d, row)) * 16


@pytest.mark.parametrize("d", [64, 128])
def test_each_row_is_a_permutation_of_its_chunks(d):
    cpr = d // 8
    for r in range(64):
        pos = sorted(c ^ swz(d, r) for c in range(cpr))
        assert pos == list(range(cpr)), r


@pytest.mark.parametrize("d", [64, 128])
def test_tile_fill_covers_every_byte_once(d):
    """Thread-chunk idx of a tile lands at byte 16 idx and carries chunk
    (idx % CPR) ^ swz(row) of row idx // CPR: a bijection onto the tile."""
    cpr = d // 8
    seen = set()
    for idx in range(64 * cpr):
        row, pos = divmod(idx, cpr)
        chunk = pos ^ swz(d, row)
        assert byte_of(d, row, chunk) == 16 * idx
        seen.add((row, chunk))
    assert len(seen) == 64 * cpr


def banks(byte, width):
    return {(byte // 4 + i) % 64 for i in range(width // 4)}


@pytest.mark.parametrize("d", [64, 128])
def test_k_fragment_reads_are_conflict_free(d):
    """ds_read_b128: lane (g, lrow) reads row 32 j + lrow, chunk 2 ks + g;
    each group of 16 lanes (256 bytes) must cover all 64 banks once."""
    ks_n = d // 16
    for j, ks in itertools.product(range(2), range(ks_n)):
        for quarter in range(4):
            used = []
            for lane in range(16 * quarter, 16 * quarter + 16):
                g, lrow = lane >> 5, lane & 31
                b = byte_of(d, 32 * j + lrow, 2 * ks + g)
                used.extend(banks(b, 16))
            assert len(used) == len(set(used)) == 64, (j, ks, quarter)


@pytest.mark.parametrize("d", [64, 128])
def test_v_transposing_reads_are_conflict_free(d):
    """ds_read_b64_tr_b16: lane reads 8 bytes of row 4 g + (tp >> 2) + 8 hi
    + 16 hh + 32 j, chunk 4 dblk + 2 ((lane >> 4) & 1) + ((tp & 3) >> 1),
    half tp & 1; each half-wave (32 lanes, 256 bytes) must cover all 64
    banks once."""
    for j, hh, hi, dblk in itertools.product(range(2), range(2), range(2), range(d // 32)):
        for half in range(2):
            used = []
            for lane in range(32 * half, 32 * half + 32):
                tp, g = lane & 15, lane >> 5
                row = 4 * g + (tp >> 2) + 8 * hi + 16 * hh + 32 * j
                chunk = 4 * dblk + 2 * ((lane >> 4) & 1) + ((tp & 3) >> 1)
                b = byte_of(d, row, chunk) + 8 * (tp & 1)
                used.extend(banks(b, 8))
            assert len(used) == len(set(used)) == 64, (j, hh, hi, dblk, half)


@pytest.mark.parametrize("d", [64, 128])
def test_read_addresses_match_the_xor_form(d):
    """The kernel forms each read address as a per-lane base XORed with a
    per-read constant; check that this equals the layout's byte offset."""
    for lane in range(64):
        g, lrow, tp = lane >> 5, lane & 31, lane & 15
        ka0 = lrow * d * 2 + ((g ^ swz(d, lrow)) * 16)
        for j, ks in itertools.product(range(2), range(d // 16)):
            assert (ka0 ^ (32 * ks)) + 64 * j * d == byte_of(d, 32 * j + lrow, 2 * ks + g)
        vrow = 4 * g + (tp >> 2)
        va0 = vrow * d * 2 + 8 * (tp & 1) + (((2 * ((lane >> 4) & 1) + ((tp & 3) >> 1)) ^ swz(d, vrow)) * 16)
        for j, hh, hi, dblk in itertools.product(range(2), range(2), range(2), range(d // 32)):
            got = (32 * j + 16 * hh) * d * 2 + 16 * d * hi + (va0 ^ (64 * dblk + 32 * hi))
            row = vrow + 8 * hi + 16 * hh + 32 * j
            chunk = 4 * dblk + 2 * ((lane >> 4) & 1) + ((tp & 3) >> 1)
            assert got == byte_of(d, row, chunk) + 8 * (tp & 1), (lane, j, hh, hi, dblk)
