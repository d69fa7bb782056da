"""The oracle's sections re-derived independently with vectorised numpy from
the definitions: code starts are the prefix sums of the code lengths; the
stream is the concatenation of the codewords MSB-first; gap[w] is the first
start at or after 64w minus 64w (or total_bits - 64w); unit_pos[u] counts the
starts before bit 4096u; sign/mantissa is (sign << 7) | mantissa."""
import numpy as np
import pytest

import df11_inputs as di
import oracle


def rederive(x, code_len):
    e = (x >> 7) & 0xFF
    ln = code_len.astype(np.int64)[e]
    starts = np.concatenate([[0], np.cumsum(ln)[:-1]]) if x.size else np.zeros(0, np.int64)
    total = int(ln.sum())
    n_windows = (total + 63) // 64
    n_units = (n_windows + 63) // 64
    # stream bits
    codes = oracle.canonical_codes(code_len).astype(np.uint64)[e]
    bits = np.zeros(512 * n_units * 8 + 128, dtype=np.uint8)
    for L in np.unique(ln):
        sel = ln == L
        for b in range(int(L)):
            bits[starts[sel] + b] = ((codes[sel] >> np.uint64(L - 1 - b)) & np.uint64(1)).astype(np.uint8)
    stream = np.packbits(bits)
    # gaps
    w0 = 64 * np.arange(n_windows, dtype=np.int64)
    idx = np.searchsorted(starts, w0, side="left")
    if starts.size:
        first = np.where(idx < starts.size, starts[np.minimum(idx, starts.size - 1)], total)
    else:
        first = np.full(n_windows, total, dtype=np.int64)
    gaps = (first - w0).astype(np.int64)
    # unit positions
    up = np.searchsorted(starts, 4096 * np.arange(n_units, dtype=np.int64), side="left").astype(np.uint64)
    up = np.concatenate([up, [x.size]]).astype(np.uint64)
    sm = (((x >> 8) & 0x80) | (x & 0x7F)).astype(np.uint8)
    return dict(total=total, n_windows=n_windows, n_units=n_units, stream=stream, gaps=gaps,
                unit_pos=up, sm=sm, starts=starts)


def check(x):
    enc = oracle.encode(x)
    r = rederive(x, enc.code_len)
    assert enc.total_bits == r["total"]
    assert enc.n_windows == r["n_windows"] and enc.n_units == r["n_units"]
    np.testing.assert_array_equal(enc.stream, r["stream"][:enc.stream.size])
    assert enc.sign_mant.size == (x.size + 15) // 16 * 16
    np.testing.assert_array_equal(enc.sign_mant[:x.size], r["sm"])
    assert not enc.sign_mant[x.size:].any()
    assert enc.gaps.size == 40 * enc.n_units + 8
    gb = np.unpackbits(enc.gaps)[:5 * enc.n_windows].reshape(-1, 5).astype(np.int64)
    fields = (gb * (1 << np.arange(4, -1, -1))).sum(axis=1) if enc.n_windows else np.zeros(0, np.int64)
    np.testing.assert_array_equal(fields, r["gaps"])
    assert not np.unpackbits(enc.gaps)[5 * enc.n_windows:].any()
    assert np.all((r["gaps"] >= 0) & (r["gaps"] <= 31))
    np.testing.assert_array_equal(enc.unit_pos, r["unit_pos"])
    # per-window code counts sum to the unit's share of outputs
    st = r["starts"]
    win_counts = np.bincount(st // 64, minlength=enc.n_windows) if st.size else np.zeros(0, np.int64)
    assert win_counts.max(initial=0) <= 64
    unit_counts = np.add.reduceat(win_counts, np.arange(0, enc.n_windows, 64)) if enc.n_windows else []
    np.testing.assert_array_equal(np.diff(enc.unit_pos.astype(np.int64)), unit_counts)
    return enc


@pytest.mark.parametrize("n", [0, 1, 7, 64, 200, 4096, 50_000, 131_071])
def test_rederive_normal(n):
    check(di.random_normal(n, 0.02, 1234 + n))


def test_rederive_c1():
    enc = check(di.generate("C1"))
    assert 2.3 < enc.total_bits / enc.n < 3.0


@pytest.mark.parametrize("seed", range(5))
def test_rederive_skewed(seed):
    check(di.skewed(60_000, 3 + 50 * seed, 1.5 - 0.2 * seed, 900 + seed))


def test_rederive_fibonacci_prefix():
    # the first 400k symbols of the Fibonacci-34 input keep long codes in play
    x = di.fibonacci_exponents()[:400_000]
    check(x)


def test_rederive_all_patterns():
    check(di.all_bf16_patterns(9))
