"""Code-length construction of the oracle pinned to mathematics: Kraft
equality, the entropy bound, brute-force optimality on tiny alphabets, a
dynamic program for optimal length-limited codes, prefix-freeness."""
import itertools
from functools import lru_cache

import numpy as np
import pytest

import oracle


def _counts(d):
    c = np.zeros(256, dtype=np.uint64)
    for e, v in d.items():
        c[e] = v
    return c


def _cost(c, ln):
    return int((c.astype(np.uint64) * ln.astype(np.uint64)).sum())


def _kraft(ln):
    ln = ln[ln > 0].astype(np.int64)
    # exact: sum 2^(63-l) == 2^63
    return sum(1 << (63 - int(l)) for l in ln)


def brute_force_min_cost(weights, cap):
    """Minimum sum w*l over all length vectors with Kraft sum <= 1 and 1<=l<=cap."""
    n = len(weights)
    w = np.asarray(weights, dtype=np.int64)
    top = min(cap, n - 1) if n > 1 else 1
    grid = np.array(list(itertools.product(range(1, top + 1), repeat=n)), dtype=np.int64)
    kraft = (2.0 ** (-grid)).sum(axis=1)
    ok = kraft <= 1.0 + 1e-12
    return int((grid[ok] * w).sum(axis=1).min())


def dp_min_cost(weights, cap):
    """Optimal length-limited prefix code cost by dynamic programming over the
    depth of a full code tree (heaviest symbols take the shallowest leaves)."""
    w = sorted(weights, reverse=True)
    n = len(w)
    if n == 1:
        return w[0]
    pre = [0]
    for v in w:
        pre.append(pre[-1] + v)
    inf = float("inf")

    @lru_cache(maxsize=None)
    def f(d, i, a):
        if i == n:
            return 0 if a == 0 else inf
        if d > cap or a > n - i or a == 0:
            return inf
        best = inf
        for k in range(0, min(a, n - i) + 1):
            rest = a - k
            if rest == 0 and i + k != n:
                continue
            sub = 0 if (rest == 0) else f(d + 1, i + k, 2 * rest)
            cand = d * (pre[i + k] - pre[i]) + sub
            if cand < best:
                best = cand
        return best

    return f(1, 0, 2)


def test_kraft_equality_and_entropy_bound_on_synthetic():
    import df11_inputs as di
    for x in [di.generate("C1"), di.random_normal(200_000, 0.02, 7),
              di.skewed(100_000, 40, 1.3, 11), di.skewed(50_000, 200, 0.7, 12)]:
        c = oracle.histogram(x)
        ln = oracle.code_lengths(c)
        assert _kraft(ln) == 1 << 63
        assert ln.max() <= 32
        h = oracle.exponent_entropy_bits(c)
        lbar = _cost(c, ln) / x.size
        assert h - 1e-12 <= lbar < h + 1


@pytest.mark.parametrize("seed", range(40))
def test_brute_force_optimal_tiny_alphabets(seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    n = int(rng.integers(2, 8))
    # small integer weights so that ties are frequent
    w = rng.integers(1, 6 if seed % 2 else 1000, size=n)
    syms = rng.choice(256, size=n, replace=False)
    c = _counts(dict(zip(map(int, syms), map(int, w))))
    ln = oracle.code_lengths(c)
    assert _cost(c, ln) == brute_force_min_cost(list(map(int, w)), cap=64)
    assert _kraft(ln) == 1 << 63


@pytest.mark.parametrize("seed", range(30))
def test_length_limited_optimal_small_caps(seed):
    rng = np.random.Generator(np.random.PCG64(1000 + seed))
    n = int(rng.integers(2, 8))
    w = [int(v) for v in (rng.integers(1, 4, size=n) if seed % 3 == 0 else
                          np.round(2.0 ** rng.uniform(0, 12, size=n)).astype(int))]
    cap = int(rng.integers(max(1, int(np.ceil(np.log2(n)))), n))
    c = _counts({e: v for e, v in zip(range(20, 20 + n), w)})
    ln = oracle.code_lengths(c, cap=cap)
    assert ln.max() <= cap
    assert _kraft(ln) == 1 << 63
    best = brute_force_min_cost(w, cap)
    assert _cost(c, ln) == best
    assert dp_min_cost(w, cap) == best
    pm = oracle.package_merge_lengths(c, cap)
    assert _cost(c, pm) == best and _kraft(pm) == 1 << 63


def test_fibonacci_34_is_capped_at_32():
    fib = [1, 1]
    while len(fib) < 34:
        fib.append(fib[-1] + fib[-2])
    c = _counts({100 + k: f for k, f in enumerate(fib)})
    assert int(c.sum()) == 14_930_351
    free = oracle.code_lengths(c, cap=63)
    assert free.max() == 33
    ln = oracle.code_lengths(c)
    assert ln.max() == 32
    assert _kraft(ln) == 1 << 63
    assert _cost(c, ln) == dp_min_cost(fib, 32)
    assert _cost(c, free) == dp_min_cost(fib, 63)
    # the package-merge lengths are monotone in the counts
    order = np.argsort(c[100:134], kind="stable")
    assert np.all(np.diff(ln[100:134][order].astype(int)) <= 0)


@pytest.mark.parametrize("seed", range(10))
def test_dp_agrees_with_package_merge_medium(seed):
    rng = np.random.Generator(np.random.PCG64(77 + seed))
    n = int(rng.integers(8, 30))
    w = [int(v) for v in np.round(2.0 ** rng.uniform(0, 20, size=n)).astype(int)]
    cap = int(rng.integers(int(np.ceil(np.log2(n))) + 1, 12))
    c = _counts({e: v for e, v in zip(range(n), w)})
    ln = oracle.code_lengths(c, cap=cap)
    assert ln.max() <= cap
    assert _cost(c, ln) == dp_min_cost(w, cap)


def _codes_as_strings(ln):
    codes = oracle.canonical_codes(ln)
    return {e: format(int(codes[e]), "0{}b".format(int(ln[e]))) for e in range(256) if ln[e]}


@pytest.mark.parametrize("seed", range(12))
def test_canonical_codes_prefix_free_and_ordered(seed):
    import df11_inputs as di
    x = di.skewed(20_000, int(5 + 20 * seed), 1.0 + 0.1 * seed, 300 + seed)
    ln = oracle.code_lengths(oracle.histogram(x))
    s = _codes_as_strings(ln)
    items = sorted(s.items(), key=lambda kv: (len(kv[1]), kv[0]))
    for (e1, a), (e2, b) in itertools.combinations(items, 2):
        assert not b.startswith(a) and not a.startswith(b)
    # canonical: in (length, exponent) order the codes, left-aligned to 64 bits, increase
    vals = [int(b, 2) << (64 - len(b)) for _, b in items]
    assert vals == sorted(vals) and len(set(vals)) == len(vals)
    assert vals[0] == 0
    # complete code: the last codeword is all ones
    assert set(items[-1][1]) == {"1"}


def test_single_symbol_and_empty():
    c = _counts({77: 12345})
    ln = oracle.code_lengths(c)
    assert ln[77] == 1 and ln.sum() == 1
    assert oracle.canonical_codes(ln)[77] == 0
    assert oracle.code_lengths(np.zeros(256, dtype=np.uint64)).sum() == 0


def test_all_256_symbols_equal_counts_are_8_bits():
    c = np.full(256, 256, dtype=np.uint64)
    ln = oracle.code_lengths(c)
    assert np.all(ln == 8)
    codes = oracle.canonical_codes(ln)
    np.testing.assert_array_equal(codes, np.arange(256, dtype=np.uint64))
