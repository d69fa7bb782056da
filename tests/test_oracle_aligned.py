"""Pins of the oracle's aligned-units format variant (ours, not the pages'):
groups of 32 codes never start in two units, the rest of a unit is zero
filler, so every unit's first weight is a multiple of 32.  Checked against a
layout derived by hand, the round trip through the oracle's unit decoder,
the invariants that define the layout, a bit-by-bit walk of every window,
and the gap rule re-applied to the pages' format (where it must give the C
oracle's gaps)."""
import numpy as np
import pytest

import df11_inputs as di
import oracle


def cyclic8(n):
    """Eight exponents in turn: equal counts, so every code is 3 bits long."""
    i = np.arange(n)
    return ((120 + (i % 8)) << 7 | (i & 0x7F)).astype(np.uint16)


def bit(stream, k):
    return (int(stream[k >> 3]) >> (7 - (k & 7))) & 1


def gap_field(gaps, w):
    return sum(bit(gaps, 5 * w + j) << (4 - j) for j in range(5))


def test_closed_form_layout():
    # 3-bit codes, groups of 96 bits: a group fits in a unit while its last code
    # (offset 93) starts before bit 4096, i.e. groups at 0, 96, ..., 96 * 41;
    # group 42 would put its last start at 4125, so bits 4032..4095 are filler.
    n = 3 * 1344 + 100
    x = cyclic8(n)
    e = oracle.encode_aligned_units(x)
    assert set(e.code_len[e.code_len > 0].tolist()) == {3}
    assert e.total_bits == 3 * 4096 + 3 * 100
    assert e.unit_pos.tolist() == [0, 1344, 2688, 4032, n]
    assert e.unit_end.tolist() == [4032, 4032, 4032, 300]
    assert all(bit(e.stream, k) == 0 for k in range(4032, 4096))
    # window 62 (bits 3968..4031): first start 3969; 63: all filler; 64: unit 1 opens
    assert [gap_field(e.gaps, w) for w in (0, 1, 62, 63, 64, 65)] == [0, 2, 1, 0, 0, 2]
    np.testing.assert_array_equal(oracle.decode_units(e), x)


def test_the_pages_format_differs_for_the_same_input():
    e = oracle.encode(cyclic8(3 * 1344 + 100))
    assert e.unit_pos[1] == 1366  # codes at 0, 3, ..., 4095


CASES = {
    "c1": lambda: di.generate("C1"),
    "ragged": lambda: di.random_normal(100_003, 0.02, 5),
    "skew_steep": lambda: di.skewed(60_000, 12, 2.5, 9),
    "skew_flat": lambda: di.skewed(60_000, 256, 0.3, 8),
    "single": lambda: di.single_exponent(10_000, 127, 1),
    "high": lambda: di.high_exponents(20_003, 7),
    "fib34": lambda: di.fibonacci_exponents()[:300_000],
    "tiny": lambda: di.random_normal(5, 0.02, 3),
    "empty": lambda: np.zeros(0, np.uint16),
}


@pytest.mark.parametrize("case", sorted(CASES))
def test_layout_invariants_and_round_trip(case):
    x = CASES[case]()
    e = oracle.encode_aligned_units(x)
    assert e.unit_pos[-1] == x.size and e.unit_end.size == e.n_units
    assert (e.unit_pos[:-1] % 32 == 0).all()
    assert (np.diff(e.unit_pos.astype(np.int64)) >= 0).all()
    if not x.size:
        return
    np.testing.assert_array_equal(oracle.decode_units(e), x)
    starts = oracle.code_starts(e, x)
    lengths = e.code_len.astype(np.int64)[(x >> 7) & 0xFF]
    unit_of = starts // 4096
    # each unit's codes start inside it, before the end of its codes
    up = e.unit_pos.astype(np.int64)
    for u in range(e.n_units):
        s = starts[up[u]:up[u + 1]]
        assert ((s // 4096) == u).all()
        end = 4096 * u + int(e.unit_end[u])
        if s.size:
            assert s[-1] < end
            # the codes are contiguous inside the unit; without filler the last may run on
            assert (np.diff(s) == lengths[up[u]:up[u + 1] - 1]).all()
        if int(e.unit_end[u]) < 4096 and u + 1 < e.n_units:
            # filler: zero bits, the last code ends where it starts, and the next
            # group would have had a code start in the next unit
            assert s[-1] + lengths[up[u + 1] - 1] == end
            assert all(bit(e.stream, k) == 0 for k in range(end, 4096 * (u + 1)))
            g = lengths[up[u + 1]:up[u + 1] + 32]
            assert end + int(g[:-1].sum()) >= 4096 * (u + 1)
            assert starts[up[u + 1]] == 4096 * (u + 1)
    # groups never start codes in two units
    grp = np.arange(x.size) // 32
    first_unit = np.zeros(grp[-1] + 1, np.int64)
    np.maximum.at(first_unit, grp, unit_of)
    assert (unit_of == first_unit[grp]).all()


def test_gap_rule_reproduces_the_pages_format():
    # the variant's gap rule with no filler (unit ends at 4096 and the stream
    # end) must give the C oracle's gaps of the pages' format
    x = di.generate("C1")
    e = oracle.encode(x)
    starts = oracle.code_starts(e, x)
    w = np.arange(e.n_windows)
    end_w = np.minimum(4096 * (w // 64 + 1), e.total_bits)
    nxt = np.searchsorted(starts, 64 * w)
    first = np.where(nxt < starts.size, starts[np.minimum(nxt, starts.size - 1)], e.total_bits)
    gap = np.where(64 * w >= end_w, 0, np.minimum(first, end_w) - 64 * w)
    assert gap.tolist() == [gap_field(e.gaps, int(k)) for k in w]


def walk_counts(e):
    """Codes that start in each window, walked bit by bit from its gap to the
    window's end or the end of its unit's codes."""
    codes = oracle.canonical_codes(e.code_len)
    table = {format(int(codes[s]), "0{}b".format(int(e.code_len[s]))): s for s in range(256) if e.code_len[s]}
    bits = "".join(format(int(b), "08b") for b in e.stream)
    out = []
    for w in range(e.n_windows):
        u = w // 64
        end = min(64 * w + 64, 4096 * u + int(e.unit_end[u]))
        pos, c = 64 * w + gap_field(e.gaps, w), 0
        while pos < end:
            for L in range(1, 33):
                if bits[pos:pos + L] in table:
                    pos += L
                    break
            else:
                raise AssertionError("no codeword")
            c += 1
        out.append(c)
    return out


@pytest.mark.parametrize("case", ["c1_part", "skew_steep", "cyclic8"])
def test_window_counts_equal_a_walk(case):
    x = {"c1_part": lambda: di.generate("C1")[:20_000], "skew_steep": lambda: di.skewed(20_000, 12, 2.5, 9),
         "cyclic8": lambda: cyclic8(3 * 1344 + 100)}[case]()
    e = oracle.encode_aligned_units(x)
    assert oracle.window_counts(e, x).tolist() == walk_counts(e)
