"""Losslessness of the oracle: decode(encode(x)) == x on the raw bits, which is
the plain definition of the result (the pages' claim of bit-for-bit identical
weights)."""
import numpy as np
import pytest

import df11_inputs as di
import oracle


def _roundtrip(x):
    enc = oracle.encode(x)
    np.testing.assert_array_equal(oracle.decode(enc), x)
    np.testing.assert_array_equal(oracle.decode_units(enc), x)
    return enc


def test_every_bf16_pattern_in_order():
    enc = _roundtrip(di.all_bf16_patterns())
    assert np.all(enc.code_len == 8)
    assert enc.total_bits == 8 * 65536


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_every_bf16_pattern_permuted(seed):
    _roundtrip(di.all_bf16_patterns(seed))


def test_every_length_one_tensor():
    allp = di.all_bf16_patterns()
    for v in allp:
        x = np.array([v], dtype=np.uint16)
        enc = oracle.encode(x)
        assert enc.total_bits == 1 and enc.n_windows == 1 and enc.n_units == 1
        assert list(enc.unit_pos) == [0, 1]
        assert oracle.decode(enc)[0] == v


def test_high_exponents_only():
    x = di.high_exponents(100_000, 5)
    enc = _roundtrip(x)
    assert set(np.nonzero(enc.code_len)[0]) <= set(range(240, 256))


def test_empty():
    enc = oracle.encode(np.zeros(0, dtype=np.uint16))
    assert enc.total_bits == 0 and enc.n_windows == 0 and enc.n_units == 0
    assert list(enc.unit_pos) == [0]
    assert enc.stream.size == 16 and not enc.stream.any()
    assert oracle.decode(enc).size == 0


@pytest.mark.parametrize("n", [1, 2, 63, 64, 65, 127, 4095, 4096, 4097, 65537, 262_143])
def test_ragged_sizes(n):
    _roundtrip(di.random_normal(n, 0.02, n))


@pytest.mark.parametrize("n", [1, 5, 4096, 4097, 300_000])
def test_single_symbol(n):
    enc = _roundtrip(di.single_exponent(n, 119, n))
    assert enc.total_bits == n


def test_fibonacci_34_roundtrip():
    x = di.fibonacci_exponents()
    enc = _roundtrip(x)
    assert enc.max_len == 32


def test_workload_c1_roundtrip():
    _roundtrip(di.generate("C1"))


@pytest.mark.parametrize("seed", range(6))
def test_skewed_roundtrip(seed):
    _roundtrip(di.skewed(150_000, 8 + 40 * seed, 0.8 + 0.25 * seed, 50 + seed))


def test_threaded_unit_decode_matches():
    x = di.random_normal(1_000_003, 0.01, 99)
    enc = oracle.encode(x)
    np.testing.assert_array_equal(oracle.decode_units(enc, threads=4), x)
