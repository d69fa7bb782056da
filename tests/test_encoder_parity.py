"""The library's host encoder against the oracle: every section byte for byte,
the decode tables against the oracle's canonical codes, and the structural
validator on corrupted sections."""
import numpy as np
import pytest

import df11_inputs as di
import huffman_decode_block_amd as hdb
import oracle
from conftest import load_golden


def assert_same_sections(x, mats=None, threads=0):
    o = oracle.encode(x)
    enc = hdb.df11_encode_block(mats if mats is not None else [x], n_threads=threads)
    s = enc.sections
    assert s.n_total == o.n and s.total_bits == o.total_bits
    assert s.n_windows == o.n_windows and s.n_units == o.n_units
    np.testing.assert_array_equal(s.code_len, o.code_len)
    np.testing.assert_array_equal(s.stream, o.stream)
    np.testing.assert_array_equal(s.sign_mant, o.sign_mant)
    np.testing.assert_array_equal(s.gaps, o.gaps)
    np.testing.assert_array_equal(s.unit_pos, o.unit_pos)
    assert s.max_code_len == o.max_len
    d = np.diff(o.unit_pos.astype(np.int64))
    assert s.max_unit_count == (int(d.max()) if d.size else 0)
    assert hdb.df11_validate(s) == hdb.DF11_OK
    c = oracle.histogram(x)
    assert abs(s.exp_entropy_bits - oracle.exponent_entropy_bits(c)) < 1e-9
    return enc


@pytest.mark.parametrize("name", ["v1_mixed_small", "v3_single_exponent", "v5_straddle_window",
                                  "v6_last_window_without_start"])
def test_golden(name):
    assert_same_sections(np.array(load_golden(name)["x"], dtype=np.uint16))


@pytest.mark.parametrize("n", [0, 1, 2, 63, 64, 65, 4095, 4096, 4097, 65_537, 1_000_003])
def test_ragged(n):
    assert_same_sections(di.random_normal(n, 0.02, 10 + n))


@pytest.mark.parametrize("threads", [1, 2, 3, 8, 16])
def test_thread_counts_give_identical_bytes(threads):
    x = di.random_normal(3_000_017, 0.015, 3)
    assert_same_sections(x, threads=threads)


def test_multi_matrix_block_matches_concatenation():
    x = di.random_normal(2_000_000, 0.02, 4)
    cuts = [0, 1, 1000, 1000, 777_777, 1_500_001, 2_000_000]
    mats = [x[a:b] for a, b in zip(cuts[:-1], cuts[1:])]
    enc = assert_same_sections(x, mats=mats)
    np.testing.assert_array_equal(enc.sections.mat_offset, np.array(cuts, dtype=np.uint64))


@pytest.mark.parametrize("case", ["all_patterns", "all_patterns_perm", "high", "single", "fib34",
                                  "many_subtables", "c1", "skew_a", "skew_b"])
def test_edge_inputs(case):
    x = {
        "all_patterns": lambda: di.all_bf16_patterns(),
        "all_patterns_perm": lambda: di.all_bf16_patterns(11),
        "high": lambda: di.high_exponents(70_000, 3),
        "single": lambda: di.single_exponent(123_457, 200, 4),
        "fib34": lambda: di.fibonacci_exponents(),
        "many_subtables": lambda: di.many_subtables(),
        "c1": lambda: di.generate("C1"),
        "skew_a": lambda: di.skewed(500_000, 60, 1.1, 8),
        "skew_b": lambda: di.skewed(500_000, 256, 0.5, 9),
    }[case]()
    assert_same_sections(x)


@pytest.mark.slow
def test_workload_c2():
    assert_same_sections(di.generate("C2"))


def _walk_tables(tables_u32, bits):
    """Decode one codeword given as a '0'/'1' string through the tables."""
    window = int((bits + "0" * 32)[:32], 2)
    e = int(tables_u32[window >> 24])
    lvl = 1
    while e & 0x80000000:
        t = (e >> 16) & 0x7FFF
        e = int(tables_u32[(t << 8) | ((window >> (24 - 8 * lvl)) & 0xFF)])
        lvl += 1
    return (e >> 23) & 0xFF, ((e >> 8) & 31) + 1, e & 31


@pytest.mark.parametrize("case", ["c1", "fib34", "many_subtables", "all_patterns", "single"])
def test_tables_decode_every_oracle_codeword(case):
    x = {"c1": lambda: di.generate("C1"), "fib34": lambda: di.fibonacci_exponents(),
         "many_subtables": lambda: di.many_subtables(), "all_patterns": lambda: di.all_bf16_patterns(),
         "single": lambda: di.single_exponent(10, 9, 1)}[case]()
    ln = oracle.code_lengths(oracle.histogram(x))
    codes = oracle.canonical_codes(ln)
    t = hdb.df11_build_tables(ln.astype(np.uint8)).view(np.uint32)
    nb, nt = hdb.df11_tables_size(ln.astype(np.uint8))
    assert nb == t.nbytes == nt * 1024 + 1024 * 4 + 2048 * 8
    for e in np.nonzero(ln)[0]:
        bits = format(int(codes[e]), "0{}b".format(int(ln[e])))
        # any continuation bits must not change the result
        for tail in ["", "1" * 31, "01" * 16]:
            sym, length, shift = _walk_tables(t, bits + tail)
            assert (sym, length) == (int(e), int(ln[e]))
            assert shift == (32 - length) & 31


def test_tables_reject_non_prefix_lengths():
    ln = np.zeros(256, dtype=np.uint8)
    ln[[1, 2, 3]] = 1  # Kraft sum 1.5
    with pytest.raises(hdb.DF11Error):
        hdb.df11_build_tables(ln)
    ln[:] = 0
    ln[5] = 33
    with pytest.raises(hdb.DF11Error):
        hdb.df11_tables_size(ln)


@pytest.mark.parametrize("what", ["unit_pos_order", "unit_pos_end", "gap_past_end", "code_len",
                                  "tables", "max_unit_count", "huge_n_total", "huge_total_bits",
                                  "total_bits_wraps"])
def test_validate_detects_corruption(what):
    x = di.random_normal(300_000, 0.02, 21)
    enc = hdb.df11_encode_block([x])
    s = enc.sections
    assert hdb.df11_validate(s) == hdb.DF11_OK
    if what == "unit_pos_order":
        s.unit_pos[3], s.unit_pos[4] = s.unit_pos[4], s.unit_pos[3]
    elif what == "unit_pos_end":
        s.unit_pos[-1] += 1
    elif what == "gap_past_end":
        # the last window holds 1 bit but its gap says 31
        w = s.n_windows - 1
        s.raw.total_bits = 64 * w + 1
        bit = 5 * w
        s.gaps[bit // 8] |= 0xFF >> (bit % 8)
        s.gaps[bit // 8 + 1] |= 0xFF
    elif what == "code_len":
        s.code_len[int(np.argmax(s.code_len))] = 40
    elif what == "tables":
        s.tables[5] ^= 1
    elif what == "max_unit_count":
        s.raw.max_unit_count += 1
    elif what == "huge_n_total":
        # sizes derived from these fields would wrap; rejected before any is read
        s.raw.n_total = 1 << 62
        s.raw.total_bits = 1 << 63
    elif what == "huge_total_bits":
        s.raw.total_bits = 33 * s.n_total
    elif what == "total_bits_wraps":
        s.raw.total_bits = (1 << 64) - 1
        s.raw.n_windows = 0
        s.raw.n_units = 0
    assert hdb.df11_validate(s) == hdb.DF11_E_FORMAT


def _greedy(bits, codes_by_bits, complete, limit):
    """Codes that start and end inside `bits` (a '0'/'1' string), greedily,
    at most `limit` of them: list of (exponent, length).  Bits that begin no
    codeword of an incomplete code read as a 1-bit code of exponent 0 (the
    tables' documented filler)."""
    out, pos = [], 0
    while pos < len(bits) and len(out) < limit:
        hit = None
        for L in range(1, len(bits) - pos + 1):
            e = codes_by_bits.get(bits[pos:pos + L])
            if e is not None:
                hit = (e, L)
                break
        if hit is None:
            if complete:
                break  # the codeword runs past the index bits
            hit = (0, 1)
        out.append(hit)
        pos += hit[1]
    return out


@pytest.mark.parametrize("case", ["c1", "fib34", "many_subtables", "all_patterns", "single", "skew"])
def test_count_and_emit_tables(case):
    x = {"c1": lambda: di.generate("C1"), "fib34": lambda: di.fibonacci_exponents(),
         "many_subtables": lambda: di.many_subtables(), "all_patterns": lambda: di.all_bf16_patterns(),
         "single": lambda: di.single_exponent(10, 9, 1), "skew": lambda: di.skewed(100_000, 90, 1.6, 5)}[case]()
    ln = oracle.code_lengths(oracle.histogram(x))
    codes = oracle.canonical_codes(ln)
    by_bits = {format(int(codes[e]), "0{}b".format(int(ln[e]))): int(e) for e in np.nonzero(ln)[0]}
    complete = len(by_bits) > 1
    t = hdb.df11_build_tables(ln.astype(np.uint8)).view(np.uint32)
    _, nt = hdb.df11_tables_size(ln.astype(np.uint8))
    count = t[nt * 256: nt * 256 + 1024]
    emit = t[nt * 256 + 1024:].reshape(2048, 2)
    for p in range(1024):
        got = _greedy(format(p, "010b"), by_bits, complete, 10)
        tb = sum(L for _, L in got)
        mask = 0
        pos = 0
        for _, L in got:
            mask |= 1 << pos
            pos += L
        want = (mask << 20) | (len(got) << 8) | tb if tb else 128  # 128: first code longer than 10 bits
        assert int(count[p]) == want, (p, hex(int(count[p])), hex(want))
    for p in range(2048):
        got = _greedy(format(p, "011b"), by_bits, complete, 4)
        lo, hi = int(emit[p, 0]), int(emit[p, 1])
        slots = [lo & 0xFFFF, lo >> 16, hi & 0xFFFF, hi >> 16]
        if not got:  # first code longer than 11 bits: t = 0, field_1 = 64
            assert lo == 64 << 16 and hi == 0
            continue
        n = len(got)
        tb = sum(L for _, L in got)
        assert slots[1] & 0x7F == n
        assert slots[0] & 0x7F == tb
        for k in range(4):
            want = (got[k][0] << 7) if k < n else 0
            assert slots[k] & 0x7F80 == want
            if k >= 2:
                assert slots[k] & 0x7F == 0
