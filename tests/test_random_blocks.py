"""Property test over seeded random blocks (six value families, log-uniform
sizes, splits into 1 to 7 matrices; `df11_inputs.random_block`): the library's
host encoder equals the oracle on every section, in the pages' format with
window counts and in the aligned-units variant, and the oracle's own unit
decoder returns the input (the method is lossless)."""
import numpy as np
import pytest

import df11_inputs as di
import huffman_decode_block_amd as hdb
import oracle

SEEDS = list(range(36))


@pytest.mark.parametrize("seed,min_n", [(s, 1) for s in SEEDS] + [(100 + s, 1 << 20) for s in range(6)])
def test_library_encoder_equals_the_oracle(seed, min_n):
    x, mats, what = di.random_block(seed, max_n=max(min_n, 1 << 20) * 4, min_n=min_n)
    o = oracle.encode(x)
    s = hdb.df11_encode_block(mats, n_threads=1 + seed % 5, window_counts=True).sections
    assert (s.n_total, s.total_bits, s.n_windows, s.n_units) == (o.n, o.total_bits, o.n_windows, o.n_units), what
    np.testing.assert_array_equal(s.code_len, o.code_len, err_msg=what)
    np.testing.assert_array_equal(s.stream, o.stream, err_msg=what)
    np.testing.assert_array_equal(s.sign_mant, o.sign_mant, err_msg=what)
    np.testing.assert_array_equal(s.gaps, o.gaps, err_msg=what)
    np.testing.assert_array_equal(s.unit_pos, o.unit_pos, err_msg=what)
    assert s.max_code_len == o.max_len, what
    decoded = oracle.decode_units(o)
    np.testing.assert_array_equal(decoded, x, err_msg=what)
    np.testing.assert_array_equal(s.counts[:o.n_windows], oracle.window_counts(o, decoded=decoded), err_msg=what)
    assert hdb.df11_validate(s) == hdb.DF11_OK, what
    starts = np.asarray(s.mat_offset)
    assert starts[0] == 0 and starts[-1] == x.size and list(np.diff(starts)) == [m.size for m in mats], what


@pytest.mark.parametrize("seed", SEEDS[::2])
def test_aligned_units_equal_the_oracle(seed):
    x, mats, what = di.random_block(seed, max_n=1 << 18)
    o = oracle.encode_aligned_units(x)
    s = hdb.df11_encode_block(mats, n_threads=1 + seed % 3, aligned_units=True).sections
    assert (s.total_bits, s.n_windows, s.n_units) == (o.total_bits, o.n_windows, o.n_units), what
    np.testing.assert_array_equal(s.stream, o.stream, err_msg=what)
    np.testing.assert_array_equal(s.gaps, o.gaps, err_msg=what)
    np.testing.assert_array_equal(s.unit_pos, o.unit_pos, err_msg=what)
    np.testing.assert_array_equal(s.unit_end, o.unit_end, err_msg=what)
    np.testing.assert_array_equal(s.sign_mant, o.sign_mant, err_msg=what)
    np.testing.assert_array_equal(oracle.decode_units(o), x, err_msg=what)
    assert hdb.df11_validate(s) == hdb.DF11_OK, what


def test_wide_sweep_pages_format():
    # many more seeds, checked in one test: every section against the oracle
    for seed in range(3000, 3300):
        x, mats, what = di.random_block(seed, max_n=1 << 18)
        o = oracle.encode(x)
        s = hdb.df11_encode_block(mats, n_threads=1 + seed % 4, window_counts=True).sections
        assert s.total_bits == o.total_bits, what
        for a, b in ((s.code_len, o.code_len), (s.stream, o.stream), (s.sign_mant, o.sign_mant), (s.gaps, o.gaps),
                     (s.unit_pos, o.unit_pos)):
            assert np.array_equal(a, b), (seed, what)
        assert np.array_equal(s.counts[:o.n_windows], oracle.window_counts(o)), (seed, what)


def test_wide_sweep_aligned_units():
    for seed in range(4000, 4100):
        x, mats, what = di.random_block(seed, max_n=1 << 16)
        o = oracle.encode_aligned_units(x)
        s = hdb.df11_encode_block(mats, aligned_units=True).sections
        assert s.total_bits == o.total_bits, what
        for a, b in ((s.stream, o.stream), (s.gaps, o.gaps), (s.unit_pos, o.unit_pos), (s.unit_end, o.unit_end),
                     (s.sign_mant, o.sign_mant)):
            assert np.array_equal(a, b), (seed, what)
