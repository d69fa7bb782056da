"""Checks that the oracle's pins have teeth: a copy of the oracle source with
one plausible mistake planted is compiled on the CPU, and the pins must fail
for it.  The unmodified oracle must pass the same pins."""
import ctypes
import os
import subprocess
import tempfile

import numpy as np
import pytest

import df11_inputs as di
import oracle
from conftest import load_golden
from test_oracle_format import check as rederive_check
from test_oracle_huffman import brute_force_min_cost

MUTANTS = {
    "huffman_tie_prefers_newer": (
        "if (best < 0 || weight[k] < weight[best]) best = k;",
        "if (best < 0 || weight[k] <= weight[best]) best = k;"),
    "canonical_no_increment": (
        "if (k > 0) c = (c + 1) << (len[order[k]] - len[order[k - 1]]);",
        "if (k > 0) c = c << (len[order[k]] - len[order[k - 1]]);"),
    "pack_lsb_first": (
        "if (bit) buf[bitpos >> 3] |= (uint8_t)(0x80u >> (bitpos & 7));",
        "if (bit) buf[bitpos >> 3] |= (uint8_t)(1u << (bitpos & 7));"),
    "pack_and_read_lsb_first": (
        ["if (bit) buf[bitpos >> 3] |= (uint8_t)(0x80u >> (bitpos & 7));",
         "return (buf[bitpos >> 3] >> (7 - (bitpos & 7))) & 1u;"],
        ["if (bit) buf[bitpos >> 3] |= (uint8_t)(1u << (bitpos & 7));",
         "return (buf[bitpos >> 3] >> (bitpos & 7)) & 1u;"]),
    "gap_strictly_after": (
        "while (next_window < s.n_windows && 64 * next_window <= bitpos) {",
        "while (next_window < s.n_windows && 64 * next_window < bitpos) {"),
    "unit_pos_strictly_after": (
        "while (next_unit < s.n_units && 4096 * next_unit <= bitpos) {",
        "while (next_unit < s.n_units && 4096 * next_unit < bitpos) {"),
    "sign_bit_misplaced": (
        "sm[i] = (uint8_t)((orc_sign_of(x[i]) << 7) | orc_mantissa_of(x[i]));",
        "sm[i] = (uint8_t)((orc_sign_of(x[i]) << 6) | orc_mantissa_of(x[i]));"),
    "decode_sign_misplaced": (
        "out[i] = (uint16_t)(((s >> 7) << 15) | (e << 7) | (s & 0x7Fu));",
        "out[i] = (uint16_t)(((s >> 7) << 14) | (e << 7) | (s & 0x7Fu));"),
    "package_first_on_ties": (
        "take_leaf = counts[sym[li]] <= pw;",
        "take_leaf = counts[sym[li]] < pw;"),
    "gap_field_lsb_first": (
        "orc_put_bit(gaps, 5 * w + (uint64_t)(4 - b), (gap_value[w] >> b) & 1u);",
        "orc_put_bit(gaps, 5 * w + (uint64_t)b, (gap_value[w] >> b) & 1u);"),
    "empty_last_window_gap_zero": (
        "gap_value[next_window] = (uint32_t)(total_bits - 64 * next_window);",
        "gap_value[next_window] = 0;"),
    "histogram_drops_lowest_exponent_bit": (
        "static unsigned orc_exponent_of(uint16_t x) { return (x >> 7) & 0xFFu; }",
        "static unsigned orc_exponent_of(uint16_t x) { return (x >> 8) & 0x7Fu; }"),
    "package_merge_takes_one_less": (
        "int take = 2 * n - 2;", "int take = 2 * n - 3;"),
}


def _pins_pass():
    """A compact run of the pins; False at the first failure."""
    try:
        for name in ["v1_mixed_small", "v3_single_exponent", "v5_straddle_window",
                     "v6_last_window_without_start"]:
            from test_oracle_golden import test_format_vector
            test_format_vector(name)
        from test_oracle_golden import test_package_merge_vector, test_tie_break_vector
        test_tie_break_vector()
        test_package_merge_vector()
        for x in [di.all_bf16_patterns(4), di.generate("C1"), di.fibonacci_exponents()[:200_000],
                  di.skewed(40_000, 30, 1.2, 5)]:
            enc = oracle.encode(x)
            np.testing.assert_array_equal(oracle.decode(enc), x)
            rederive_check(x)
        rng = np.random.Generator(np.random.PCG64(3))
        for _ in range(6):
            n = int(rng.integers(2, 7))
            w = [int(v) for v in rng.integers(1, 9, size=n)]
            c = np.zeros(256, dtype=np.uint64)
            c[40:40 + n] = w
            ln = oracle.code_lengths(c)
            assert int((ln.astype(np.uint64) * c).sum()) == brute_force_min_cost(w, 64)
        return True
    except (AssertionError, ValueError, IndexError):
        return False


def _with_library(path):
    saved = (oracle._LIB_PATH, oracle._lib)
    oracle._LIB_PATH, oracle._lib = path, None
    try:
        return _pins_pass()
    finally:
        oracle._LIB_PATH, oracle._lib = saved


def test_unmodified_oracle_passes_the_pins():
    assert _pins_pass()


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name, tmp_path):
    src = open(oracle._SRC).read()
    old, new = MUTANTS[name]
    olds, news = (old, new) if isinstance(old, list) else ([old], [new])
    for o, n in zip(olds, news):
        assert src.count(o) == 1, f"mutation site not found: {o}"
        src = src.replace(o, n)
    c_path = tmp_path / "mutant.c"
    c_path.write_text(src)
    so_path = str(tmp_path / f"liboracle_mutant_{name}.so")
    subprocess.check_call(["gcc", "-O1", "-std=c99", "-shared", "-fPIC", "-pthread", str(c_path),
                           "-o", so_path])
    assert not _with_library(so_path), f"the pins did not catch mutant {name}"
