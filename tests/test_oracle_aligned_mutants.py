"""The aligned-units pins have teeth: the oracle's layout and encoding
functions, each with one plausible mistake planted (a source edit, run in the
oracle's own namespace), must fail at least one of the pins of
test_oracle_aligned.py; the unmodified functions pass them all."""
import inspect

import numpy as np
import pytest

import df11_inputs as di
import oracle
import test_oracle_aligned as pins

MUTANTS = {
    "fits_when_last_start_is_on_the_boundary": (
        "aligned_layout", "if pos + offs[-1] >= (u + 1) * UNIT_BITS:", "if pos + offs[-1] > (u + 1) * UNIT_BITS:"),
    "fit_tested_on_the_first_code": (
        "aligned_layout", "if pos + offs[-1] >= (u + 1) * UNIT_BITS:", "if pos + offs[0] >= (u + 1) * UNIT_BITS:"),
    "no_jump_over_the_filler": (
        "aligned_layout", "            pos = (u + 1) * UNIT_BITS\n", "            pos = pos\n"),
    "groups_of_16": (
        "aligned_layout", "for g0 in range(0, n, GROUP):", "for g0 in range(0, n, 16):"),
    "last_unit_ends_at_4096": (
        "aligned_layout", "ends.get(u, min((u + 1) * UNIT_BITS, total_bits))", "ends.get(u, (u + 1) * UNIT_BITS)"),
    "gap_of_a_filler_window_not_zero": (
        "encode_aligned_units", "gap = np.where(64 * w >= end_w, 0, np.minimum(first, end_w) - 64 * w)",
        "gap = np.where(64 * w >= end_w, 1, np.minimum(first, end_w) - 64 * w)"),
    "gap_ignores_the_unit_end": (
        "encode_aligned_units", "gap = np.where(64 * w >= end_w, 0, np.minimum(first, end_w) - 64 * w)",
        "gap = np.where(64 * w >= end_w, 0, np.minimum(first, first) - 64 * w)"),
    "filler_bits_set": (
        "encode_aligned_units", "    stream = np.packbits(bits)\n",
        "    bits[ends_abs[0]:min(4096, 8 * (512 * n_units))] = 1\n    stream = np.packbits(bits)\n"),
    "unit_pos_counts_starts_up_to_the_boundary": (
        "encode_aligned_units", "np.searchsorted(starts, UNIT_BITS * np.arange(n_units, dtype=np.int64))",
        "np.searchsorted(starts, UNIT_BITS * np.arange(n_units, dtype=np.int64), side='right')"),
}


def planted(monkeypatch, fn_name, old, new):
    src = inspect.getsource(getattr(oracle, fn_name))
    assert src.count(old) == 1, (fn_name, old)
    ns = dict(vars(oracle))
    exec(compile(src.replace(old, new), f"<mutant {fn_name}>", "exec"), ns)
    monkeypatch.setattr(oracle, fn_name, ns[fn_name])


def all_pins_pass() -> bool:
    try:
        pins.test_closed_form_layout()
        for case in ("c1", "skew_steep", "fib34", "single"):
            pins.test_layout_invariants_and_round_trip(case)
        pins.test_window_counts_equal_a_walk("cyclic8")
    except (AssertionError, ValueError, IndexError):
        return False
    return True


def test_the_oracle_passes_the_pins():
    assert all_pins_pass()


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_each_mutant_fails_a_pin(monkeypatch, name):
    fn, old, new = MUTANTS[name]
    planted(monkeypatch, fn, old, new)
    assert not all_pins_pass(), f"mutant {name} passes every pin"
