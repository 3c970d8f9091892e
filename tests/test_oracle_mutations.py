"""Planted mistakes in the CPU oracle must make its pins fail.

Each case swaps one oracle step for a plausible wrong variant (on the CPU,
through monkeypatch) and checks that at least one pin of
test_oracle_pins.py raises.  This shows the pins are not vacuous.
"""
import numpy as np
import pytest

import oracle
import oracle.method as oz
from tests import test_oracle_pins as pins

_orig = {name: getattr(oz, name) for name in
         ["centered_residue", "crt", "scale_truncate", "fast_exponents",
          "accu_bound_inputs", "_accu_d", "residue_product", "inverse_scale", "moduli"]}


def _nonneg_residue(xp, m):
    r = _orig["centered_residue"](xp, m)
    return np.where(r < 0, r + m, r)


def _unsigned_residue(xp, m):
    return _orig["centered_residue"](np.abs(xp), m)


def _crt_drops_last(residues, s):
    mods = _orig["moduli"](s)
    x = _orig["crt"](residues[:-1], s - 1) if s > 2 else _orig["crt"](residues, s)
    return x if s > 2 else x + 0 * mods[0]


def _round_not_trunc(rows, d):
    rows = np.asarray(rows, dtype=np.float64)
    return np.round(np.ldexp(rows, np.asarray(d, dtype=np.int64)[:, None].astype(np.int32)))


def _fast_plus_one(rows, s):
    d, e, S = _orig["fast_exponents"](rows, s)
    return np.where(np.array([x is not None for x in e], dtype=bool), d + 1, d), e, S


def _fast_minus_one(rows, s):
    d, e, S = _orig["fast_exponents"](rows, s)
    return np.where(np.array([x is not None for x in e], dtype=bool), d - 1, d), e, S


def _accu_round_down(rows):
    e, abar = _orig["accu_bound_inputs"](rows)
    rows = np.asarray(rows, dtype=np.float64)
    out = abar.copy()
    for i, ei in enumerate(e):
        if ei is not None:
            out[i] = np.floor(np.ldexp(np.abs(rows[i]), oracle.Q_BITS - ei)).astype(np.int64)
    return e, out


def _accu_d_plus_one(e_list, peaks, s):
    d = _orig["_accu_d"](e_list, peaks, s)
    return np.where(np.array([x is not None for x in e_list], dtype=bool), d + 1, d)


def _accu_d_minus_one(e_list, peaks, s):
    d = _orig["_accu_d"](e_list, peaks, s)
    return np.where(np.array([x is not None for x in e_list], dtype=bool), d - 1, d)


def _accu_d_zero_peak_unscaled(e_list, peaks, s):
    d = _orig["_accu_d"](e_list, peaks, s)
    return np.where(np.asarray(peaks, dtype=np.int64) == 0, 0, d)


def _product_reversed_k(at, bt):
    return _orig["residue_product"](np.asarray(at)[:, ::-1], bt)


def _inverse_scale_wrong_sign(x, d, b):
    return _orig["inverse_scale"](x, -np.asarray(d), -np.asarray(b))


CASES = [
    ("centered_residue", _nonneg_residue, lambda g: pins.test_centered_residue_definition()),
    ("centered_residue", _unsigned_residue, lambda g: pins.test_centered_residue_definition()),
    ("crt", _crt_drops_last, lambda g: pins.test_crt_recovers_exact_integer_product("fast", 14, 1.0)),
    ("scale_truncate", _round_not_trunc, lambda g: pins.test_identity_right_factor_closed_form(14)),
    ("fast_exponents", _fast_plus_one, lambda g: pins.test_fast_exponent_sound_and_near_maximal(14)),
    ("fast_exponents", _fast_minus_one, lambda g: pins.test_fast_exponent_sound_and_near_maximal(14)),
    ("accu_bound_inputs", _accu_round_down, lambda g: pins.test_accu_bound_inputs_round_upward(14)),
    ("_accu_d", _accu_d_plus_one, lambda g: pins.test_eq18_equal_budget_on_flat_lines_accu()),
    ("_accu_d", _accu_d_minus_one, lambda g: pins.test_eq18_equal_budget_on_flat_lines_accu()),
    ("_accu_d", _accu_d_plus_one, lambda g: pins.test_accu_exponent_maximal_against_bruteforce(14)),
    ("_accu_d", _accu_d_minus_one, lambda g: pins.test_accu_exponent_maximal_against_bruteforce(14)),
    ("_accu_d", _accu_d_zero_peak_unscaled, lambda g: pins.test_accu_nonzero_line_with_zero_bound_peak(14)),
    ("residue_product", _product_reversed_k, lambda g: pins.test_residue_product_bruteforce()),
    ("inverse_scale", _inverse_scale_wrong_sign,
     lambda g: pins.test_small_integer_inputs_give_exact_product("fast", 14)),
]


@pytest.mark.parametrize("name,wrong,pin", CASES, ids=[f"{c[0]}-{c[1].__name__}" for c in CASES])
def test_planted_mistake_is_caught(monkeypatch, golden_dir, name, wrong, pin):
    monkeypatch.setattr(oz, name, wrong)
    if hasattr(oracle, name):
        monkeypatch.setattr(oracle, name, wrong)
    with pytest.raises(Exception):
        pin(golden_dir)


def test_unplanted_pins_pass(golden_dir):
    for _, _, pin in CASES:
        pin(golden_dir)
