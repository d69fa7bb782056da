"""Pins of the oracle's per-window code counts (the counting-free format
variant).  The oracle derives them from code start positions; here they are
checked against values derived by hand (golden vectors), against a bit-by-bit
walk of every window from its gap (the decoder's view), and against the
stored unit positions."""
import numpy as np
import pytest

import df11_inputs as di
import huffman_decode_block_amd as hdb
import oracle
from conftest import load_golden


def walk_counts(enc) -> list:
    """For each window, start at its gap and take codewords one bit pattern at
    a time (prefix match against the canonical code) until the window end or
    the end of the stream."""
    codes = oracle.canonical_codes(enc.code_len)
    table = {format(int(codes[e]), "0{}b".format(int(enc.code_len[e]))): e
             for e in range(256) if enc.code_len[e]}
    bits = "".join(format(int(b), "08b") for b in enc.stream)
    gbits = "".join(format(int(b), "08b") for b in enc.gaps)
    out = []
    for w in range(enc.n_windows):
        pos = 64 * w + int(gbits[5 * w:5 * w + 5], 2)
        end = min(64 * w + 64, enc.total_bits)
        c = 0
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


@pytest.mark.parametrize("name,want", [("v1_mixed_small", [8]), ("v3_single_exponent", [5]),
                                       ("v5_straddle_window", None), ("v6_last_window_without_start", None)])
def test_counts_of_golden_vectors(name, want):
    g = load_golden(name)
    x = np.array(g["x"], dtype=np.uint16)
    want = want if want is not None else g["window_code_counts"]
    enc = oracle.encode(x)
    assert oracle.window_counts(enc).tolist() == want
    assert walk_counts(enc) == want


SMALL = {
    "c1": lambda: di.generate("C1"),
    "skew_steep": lambda: di.skewed(20_000, 12, 2.5, 9),
    "skew_flat": lambda: di.skewed(20_000, 256, 0.3, 8),
    "single": lambda: di.single_exponent(3000, 127, 1),
    "high": lambda: di.high_exponents(5_003, 7),
    "ragged_65": lambda: di.random_normal(65, 0.02, 3),
}


@pytest.mark.parametrize("case", sorted(SMALL))
def test_counts_equal_a_walk_of_every_window(case):
    enc = oracle.encode(SMALL[case]())
    assert oracle.window_counts(enc).tolist() == walk_counts(enc)


@pytest.mark.parametrize("case", ["c2", "fib34"])
def test_counts_sum_to_the_unit_positions(case):
    x = di.generate("C2") if case == "c2" else di.fibonacci_exponents()
    enc = oracle.encode(x)
    c = oracle.window_counts(enc).astype(np.int64)
    assert c.max() <= 64
    pad = np.zeros(64 * enc.n_units, np.int64)
    pad[:c.size] = c
    np.testing.assert_array_equal(pad.reshape(-1, 64).sum(1), np.diff(enc.unit_pos.astype(np.int64)))


@pytest.mark.parametrize("case", sorted(SMALL) + ["fib34", "many_subtables"])
def test_library_counts_equal_the_oracle(case):
    x = {"fib34": di.fibonacci_exponents, "many_subtables": di.many_subtables}.get(case, SMALL.get(case))()
    enc = hdb.df11_encode_block([x], window_counts=True)
    s = enc.sections
    want = oracle.window_counts(oracle.encode(x))
    assert s.counts.size == 64 * s.n_units
    np.testing.assert_array_equal(s.counts[:s.n_windows], want)
    assert not s.counts[s.n_windows:].any()
    assert hdb.df11_validate(s) == hdb.DF11_OK
    # the other sections do not change with the option
    plain = hdb.df11_encode_block([x]).sections
    assert plain.counts is None
    for a, b in [(s.stream, plain.stream), (s.gaps, plain.gaps), (s.unit_pos, plain.unit_pos),
                 (s.sign_mant, plain.sign_mant), (s.tables, plain.tables)]:
        np.testing.assert_array_equal(a, b)


def test_validate_rejects_inconsistent_counts():
    x = di.generate("C1")
    enc = hdb.df11_encode_block([x], window_counts=True)
    s = enc.sections
    w = int(np.nonzero(s.counts)[0][0])
    s.counts[w] += 1  # the unit's counts no longer sum to its weights
    assert hdb.df11_validate(s) == hdb.DF11_E_FORMAT
    s.counts[w] -= 1
    s.counts[-1] = 1  # a padding window with a count
    assert hdb.df11_validate(s) == hdb.DF11_E_FORMAT
    s.counts[-1] = 0
    assert hdb.df11_validate(s) == hdb.DF11_OK


def test_unknown_encoder_flags_are_rejected():
    x = di.generate("C1")
    views = (hdb.df11_bf16_view * 1)()
    views[0].data = x.ctypes.data
    views[0].numel = x.size
    h = hdb._vp()
    assert hdb.lib().df11_encode_block_ex(views, 1, 0, 4, hdb.ctypes.byref(h)) == hdb.DF11_E_INVALID_ARG
