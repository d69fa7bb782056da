"""Host side of the GPU encoder: its plan (code lengths and every section
size, from the 256 exponent counts) equals what the host encoder produces for
the same weights."""
import numpy as np
import pytest

import df11_inputs as di
import huffman_decode_block_amd as hdb
import oracle

CASES = {
    "c1": lambda: di.generate("C1"),
    "fib34": lambda: di.fibonacci_exponents(),
    "many_subtables": lambda: di.many_subtables(),
    "single": lambda: di.single_exponent(1000, 127, 1),
    "all_patterns": lambda: di.all_bf16_patterns(),
    "ragged_1": lambda: di.random_normal(1, 0.02, 1),
}


@pytest.mark.parametrize("case", sorted(CASES))
@pytest.mark.parametrize("flags", [0, hdb.DF11_ENCODE_WINDOW_COUNTS])
def test_plan_matches_the_host_encoder(case, flags):
    x = CASES[case]()
    hist = np.bincount((x >> 7) & 0xFF, minlength=256).astype(np.uint64)
    np.testing.assert_array_equal(hist, oracle.histogram(x))
    plan = hdb.df11_gpu_plan_build(hist, flags)
    s = hdb.df11_encode_block([x], window_counts=bool(flags)).sections
    assert bytes(plan.code_len) == bytes(s.code_len)
    for f in ("n_total", "total_bits", "n_windows", "n_units", "max_code_len", "n_tables", "n_symbols"):
        assert getattr(plan, f) == getattr(s, f), f
    assert plan.stream_bytes == s.raw.stream_bytes
    assert plan.sign_mant_bytes == s.raw.sign_mant_bytes
    assert plan.gaps_bytes == s.raw.gaps_bytes
    assert plan.tables_bytes == s.raw.tables_bytes
    assert plan.counts_bytes == s.raw.counts_bytes
    assert plan.unit_pos_bytes == 8 * (s.n_units + 1)
    assert plan.workspace_bytes > 0


def test_plan_rejects_bad_arguments():
    with pytest.raises(hdb.DF11Error):
        hdb.df11_gpu_plan_build(np.zeros(256, np.uint64), 2)  # unknown flag
    with pytest.raises(ValueError):
        hdb.df11_gpu_plan_build(np.zeros(255, np.uint64))


def test_plan_refuses_histograms_beyond_any_block():
    big = np.zeros(256, np.uint64)
    big[127] = 1 << 49
    with pytest.raises(hdb.DF11Error):
        hdb.df11_gpu_plan_build(big)
    # counts whose sum wraps around 2^64
    wrap = np.zeros(256, np.uint64)
    wrap[10] = wrap[11] = np.uint64(1 << 63)
    with pytest.raises(hdb.DF11Error):
        hdb.df11_gpu_plan_build(wrap)


def test_empty_histogram_gives_an_empty_block():
    plan = hdb.df11_gpu_plan_build(np.zeros(256, np.uint64))
    assert plan.n_total == 0 and plan.total_bits == 0 and plan.n_units == 0


def test_encode_refuses_plans_beyond_any_block_before_any_launch():
    # a plan whose sizes all follow from its n_total and total_bits, but with
    # more weights than any block holds; the pointers are placeholders that are
    # never dereferenced (the call returns before any HIP call)
    import ctypes
    x = di.random_normal(10_000, 0.02, 3)
    plan = hdb.df11_gpu_plan_build(oracle.histogram(x).astype(np.uint64))
    big = hdb.df11_gpu_plan.from_buffer_copy(plan)
    big.n_total = 1 << 50
    big.sign_mant_bytes = (big.n_total + 15) // 16 * 16
    fake = 1 << 20
    st = hdb.lib().df11_gpu_encode(ctypes.byref(big), fake, fake, fake, fake, fake, fake, None, fake, None)
    assert st == hdb.DF11_E_INVALID_ARG
