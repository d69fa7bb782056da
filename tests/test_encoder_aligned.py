"""The library's host encoder with DF11_ENCODE_ALIGNED_UNITS equals the
oracle's aligned-units variant byte for byte on every section (the oracle's
variant is pinned in test_oracle_aligned.py), with and without window counts,
for any thread count and matrix split; the validator accepts it and rejects
what breaks the layout."""
import numpy as np
import pytest

import df11_inputs as di
import huffman_decode_block_amd as hdb
import oracle


def cyclic8(n):
    i = np.arange(n)
    return ((120 + (i % 8)) << 7 | (i & 0x7F)).astype(np.uint16)


CASES = {
    "cyclic8": lambda: cyclic8(3 * 1344 + 100),
    "c1": lambda: di.generate("C1"),
    "ragged": lambda: di.random_normal(100_003, 0.02, 5),
    "skew_steep": lambda: di.skewed(60_000, 12, 2.5, 9),
    "skew_flat": lambda: di.skewed(60_000, 256, 0.3, 8),
    "single": lambda: di.single_exponent(10_000, 127, 1),
    "high": lambda: di.high_exponents(20_003, 7),
    "fib34": lambda: di.fibonacci_exponents()[:300_000],
    "all_patterns": lambda: di.all_bf16_patterns(3),
    "tiny": lambda: di.random_normal(5, 0.02, 3),
    "one": lambda: di.random_normal(1, 0.02, 3),
}


def check_equal(s, o):
    assert s.total_bits == o.total_bits and s.n_windows == o.n_windows and s.n_units == o.n_units
    assert bytes(s.code_len) == bytes(o.code_len)
    np.testing.assert_array_equal(s.stream, o.stream)
    np.testing.assert_array_equal(s.gaps, o.gaps)
    np.testing.assert_array_equal(s.unit_pos, o.unit_pos)
    np.testing.assert_array_equal(s.unit_end, o.unit_end)
    np.testing.assert_array_equal(s.sign_mant, o.sign_mant)


@pytest.mark.parametrize("case", sorted(CASES))
def test_sections_equal_the_oracle(case):
    x = CASES[case]()
    o = oracle.encode_aligned_units(x)
    s = hdb.df11_encode_block([x], aligned_units=True).sections
    check_equal(s, o)
    assert s.counts is None
    assert hdb.df11_validate(s) == hdb.DF11_OK
    assert s.max_unit_count == int(np.diff(o.unit_pos.astype(np.int64)).max())


@pytest.mark.parametrize("threads", [1, 3, 8])
def test_threads_and_matrix_splits(threads):
    x = di.random_normal(300_001, 0.02, 11)
    o = oracle.encode_aligned_units(x)
    for split in ([x], [x[:70_001], x[70_001:70_001], x[70_001:]], [x[i:i + 4097] for i in range(0, x.size, 4097)]):
        s = hdb.df11_encode_block(split, n_threads=threads, aligned_units=True).sections
        check_equal(s, o)


@pytest.mark.parametrize("case", ["c1", "skew_steep", "cyclic8", "fib34"])
def test_with_window_counts(case):
    x = CASES[case]()
    o = oracle.encode_aligned_units(x)
    s = hdb.df11_encode_block([x], window_counts=True, aligned_units=True).sections
    check_equal(s, o)
    want = oracle.window_counts(o, x)
    np.testing.assert_array_equal(s.counts[:s.n_windows], want)
    assert not s.counts[s.n_windows:].any()
    assert hdb.df11_validate(s) == hdb.DF11_OK


def test_the_pages_format_is_unchanged_by_the_option_being_off():
    x = di.generate("C1")
    a = hdb.df11_encode_block([x]).sections
    o = oracle.encode(x)
    assert a.unit_end is None
    np.testing.assert_array_equal(a.stream, o.stream)
    np.testing.assert_array_equal(a.unit_pos, o.unit_pos)


def test_validate_rejects_a_broken_layout():
    x = cyclic8(3 * 1344 + 100)
    s = hdb.df11_encode_block([x], aligned_units=True).sections
    assert hdb.df11_validate(s) == hdb.DF11_OK
    # a nonzero filler bit (bits 4032..4095 of unit 0)
    s.stream[4040 >> 3] ^= 0x01
    assert hdb.df11_validate(s) == hdb.DF11_E_FORMAT
    s.stream[4040 >> 3] ^= 0x01
    # a unit end past its unit, and one that is 0
    for bad in (4097, 0):
        keep = int(s.unit_end[1])
        s.unit_end[1] = bad
        assert hdb.df11_validate(s) == hdb.DF11_E_FORMAT
        s.unit_end[1] = keep
    # the last unit's end must be the stream's end
    s.unit_end[-1] -= 1
    assert hdb.df11_validate(s) == hdb.DF11_E_FORMAT
    s.unit_end[-1] += 1
    assert hdb.df11_validate(s) == hdb.DF11_OK


def test_validate_rejects_a_unit_position_off_the_32_grid():
    x = di.generate("C1")
    s = hdb.df11_encode_block([x], aligned_units=True).sections
    assert s.n_units > 2
    s.unit_pos[1] += 1
    assert hdb.df11_validate(s) == hdb.DF11_E_FORMAT


def test_gpu_plan_refuses_the_aligned_layout():
    with pytest.raises(hdb.DF11Error):
        hdb.df11_gpu_plan_build(np.bincount(np.zeros(10, np.int64), minlength=256).astype(np.uint64),
                                hdb.DF11_ENCODE_ALIGNED_UNITS)
