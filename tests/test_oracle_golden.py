"""The oracle against vectors derived by hand from the pages' format description
and the stated readings (fixtures under tests/golden, each with its citation
and derivation)."""
import numpy as np
import pytest

import oracle
from conftest import load_golden

FORMAT_VECTORS = ["v1_mixed_small", "v3_single_exponent", "v5_straddle_window",
                  "v6_last_window_without_start"]


def _len_dict(code_len):
    return {str(e): int(code_len[e]) for e in range(256) if code_len[e]}


@pytest.mark.parametrize("name", FORMAT_VECTORS)
def test_format_vector(name):
    d = load_golden(name)
    x = np.array(d["x"], dtype=np.uint16)
    enc = oracle.encode(x)
    assert _len_dict(enc.code_len) == d["code_len"]
    codes = oracle.canonical_codes(enc.code_len)
    for e, bits in d["codes"].items():
        e = int(e)
        assert format(int(codes[e]), "0{}b".format(int(enc.code_len[e]))) == bits
    assert enc.total_bits == d["total_bits"]
    assert enc.n_windows == d["n_windows"]
    assert enc.n_units == d["n_units"]
    nb = (enc.total_bits + 7) // 8
    assert enc.stream[:nb].tobytes().hex() == d["stream_hex"]
    assert not enc.stream[nb:].any()
    assert enc.stream.size == 512 * enc.n_units + 16
    assert enc.sign_mant[:x.size].tobytes().hex() == d["sign_mant_hex"]
    assert not enc.sign_mant[x.size:].any()
    assert list(map(int, enc.unit_pos)) == d["unit_pos"]
    if "gaps_hex" in d:
        assert enc.gaps[:len(d["gaps_hex"]) // 2].tobytes().hex() == d["gaps_hex"]
    # gap fields read back MSB-first, 5 bits each
    bits = np.unpackbits(enc.gaps)
    fields = [int("".join(map(str, bits[5 * w:5 * w + 5])), 2) for w in range(enc.n_windows)]
    assert fields == d["gaps"]
    np.testing.assert_array_equal(oracle.decode(enc), x)
    np.testing.assert_array_equal(oracle.decode_units(enc), x)


def test_tie_break_vector():
    d = load_golden("v2_tie_break_counts")
    c = np.zeros(256, dtype=np.uint64)
    for e, v in d["counts"].items():
        c[int(e)] = v
    ln = oracle.code_lengths(c)
    assert _len_dict(ln) == d["code_len"]
    codes = oracle.canonical_codes(ln)
    for e, bits in d["codes"].items():
        assert format(int(codes[int(e)]), "0{}b".format(int(ln[int(e)]))) == bits


def test_package_merge_vector():
    d = load_golden("v4_package_merge_cap3")
    c = np.zeros(256, dtype=np.uint64)
    for e, v in d["counts"].items():
        c[int(e)] = v
    assert _len_dict(oracle.code_lengths(c)) == d["code_len_unrestricted"]
    capped = oracle.code_lengths(c, cap=d["cap"])
    assert _len_dict(capped) == d["code_len_capped"]
    assert int((capped.astype(np.uint64) * c).sum()) == d["cost_capped"]
