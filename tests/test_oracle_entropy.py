"""Pins of the oracle's exponent-entropy statistic (the Shannon entropy of the
exponent distribution, which the hada.io summary of the DFloat11 paper uses in
section "La marge de compression restante dans l'exposant BFloat16" to show
that the exponent carries far fewer bits than its 8).

The entropy has closed forms on small distributions, so the pins are exact
values, not only the one-bit window H <= mean code length < H + 1:
  - counts {4, 2, 1, 1} (the exponents of hand vector V1): 1.75 bits;
  - 2^k equal counts: k bits, whatever the common count;
  - counts {1, 3}: 2 - (3/4) log2 3 bits;
  - one symbol, or no weights: 0 bits;
  - scaling every count by the same factor leaves it unchanged; zero counts
    add nothing.
Planted mistakes in a copy of the function (count-1 symbols dropped, natural
or base-10 logarithm, unnormalised probabilities, a lost sign) must fail them.
"""
import inspect
import math

import numpy as np
import pytest

import oracle
from conftest import load_golden

EXACT = 1e-12


def pins_hold(entropy) -> list:
    """Returns the pins that `entropy` breaks (empty when all hold)."""
    failed = []

    def check(name, got, want):
        if not (isinstance(got, float) and math.isfinite(got) and abs(got - want) <= EXACT):
            failed.append(f"{name}: {got!r} != {want!r}")

    v1 = np.array(load_golden("v1_mixed_small")["x"], dtype=np.uint16)
    check("V1 histogram", entropy(oracle.histogram(v1)), 1.75)
    check("V1 counts", entropy([4, 2, 1, 1]), 1.75)
    for k in range(0, 9):
        for c in (1, 3, 1000):
            check(f"2^{k} symbols of count {c}", entropy([c] * (1 << k)), float(k))
    check("{1,3}", entropy([1, 3]), 2.0 - 0.75 * math.log2(3.0))
    check("{3,1} in a 256-bin histogram", entropy([0] * 40 + [3] + [0] * 100 + [1] + [0] * 114),
          2.0 - 0.75 * math.log2(3.0))
    check("one symbol", entropy([0, 17, 0]), 0.0)
    check("no weights", entropy([0] * 256), 0.0)
    base = [5, 1, 1, 2, 9, 1]
    ref = entropy(base)
    check("scaled x7", entropy([7 * c for c in base]), ref)
    return failed


def test_oracle_entropy_closed_forms():
    assert pins_hold(oracle.exponent_entropy_bits) == []


MUTANTS = {
    "drops_count_one_symbols": ("p = c[c > 0] / tot", "p = c[c > 1] / tot"),
    "natural_log": ("np.log2(p)", "np.log(p)"),
    "log10": ("np.log2(p)", "np.log10(p)"),
    "unnormalised": ("p = c[c > 0] / tot", "p = c[c > 0]"),
    "lost_sign": ("return float(-(p * np.log2(p)).sum())", "return float((p * np.log2(p)).sum())"),
    "total_of_others": ("p = c[c > 0] / tot", "p = c[c > 0] / (tot - c.max() + 1)"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_entropy_pins_catch_planted_mistakes(name):
    src = inspect.getsource(oracle.exponent_entropy_bits)
    old, new = MUTANTS[name]
    assert old in src, f"mutation site for {name} not found"
    ns = {"np": np}
    exec(src.replace(old, new), ns)
    assert pins_hold(ns["exponent_entropy_bits"]), f"mutant {name} passes every entropy pin"
