"""Plant mistakes in copies of the oracle: every mutant must fail a pin.

Each mutant is the oracle's source with one plausible slip applied as a text
substitution (a dropped term, a wrong sign, a transposed operand or index, a
different reading of the page's pseudocode). This shows the pins would catch
such a slip in the oracle itself.
"""
import inspect
import types

import numpy as np
import pytest

import oracle.q8_oracle as Q8
import oracle.wkv7_oracle as ORC
from tests import oracle_pins as P
from tests import q8_pins as QP

MUTANTS = {
    "drop_delta_term": ("+ sa[..., :, None] * b[..., None, :]", ""),
    "decay_before_delta": ("sa = (S * a[..., None, :]).sum(axis=-1)",
                           "sa = (S * w[..., None, :] * a[..., None, :]).sum(axis=-1)"),
    "k_in_place_of_b": ("sa[..., :, None] * b[..., None, :]",
                        "sa[..., :, None] * k[..., None, :]"),
    "readout_before_update": ("o = (S_next * r[..., None, :])",
                              "o = (S * r[..., None, :])"),
    "readout_transposed": ("o = (S_next * r[..., None, :]).sum(axis=-1)",
                           "o = (S_next * r[..., :, None]).sum(axis=-2)"),
    "outer_product_transposed": ("v[..., :, None] * k[..., None, :]",
                                 "k[..., :, None] * v[..., None, :]"),
    "delta_sign": ("+ sa[..., :, None] * b[..., None, :]",
                   "- sa[..., :, None] * b[..., None, :]"),
    "sa_transposed": ("sa = (S * a[..., None, :]).sum(axis=-1)",
                      "sa = (S * a[..., :, None]).sum(axis=-2)"),
    "decay_on_rows": ("S * w[..., None, :]", "S * w[..., :, None]"),
    "stale_decay_index": ("o[t], S = wkv7_step(S, r[t], w[t],",
                          "o[t], S = wkv7_step(S, r[t], w[max(t - 1, 0)],"),
    "a_b_swapped": ("sa = (S * a[..., None, :]).sum(axis=-1)",
                    "sa = (S * b[..., None, :]).sum(axis=-1)"),
}


def _mutant(name):
    src = inspect.getsource(ORC)
    old, new = MUTANTS[name]
    assert src.count(old) >= 1, f"mutation anchor for {name} not found"
    src = src.replace(old, new, 1)
    mod = types.ModuleType(f"oracle_mutant_{name}")
    exec(compile(src, f"<mutant {name}>", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    mod = _mutant(name)
    failures = []
    for pin in P.ALL_PINS:
        try:
            with np.errstate(all="ignore"):
                pin(mod.wkv7_sequence)
        except (AssertionError, FloatingPointError, ValueError,
                np.linalg.LinAlgError):
            failures.append(pin.__name__)
    assert failures, f"mutant {name} passed every pin"


Q8_MUTANTS = {
    "scale_over_128": ("m / np.float32(127.0)", "m / np.float32(128.0)"),
    "bankers_rounding": ("r = fl + (frac >= np.float32(0.5))",
                         "r = fl + (frac > np.float32(0.5))"),
    "round_by_adding_half": ("fl = np.floor(a)", "fl = np.floor(a + np.float32(0.5)) - np.float32(0.5)"),
    "truncate_codes": ("q[nz] = roundf(quot).astype(np.int8)",
                       "q[nz] = np.trunc(quot).astype(np.int8)"),
    "scale_from_sum": ("m = np.max(np.abs(x), axis=1)",
                       "m = np.sum(np.abs(x), axis=1) / x.shape[1] * 3"),
    "scales_swapped": ("* w_scale.astype(np.float64)[None, :] \\\n        * x_scale.astype(np.float64)[:, None]",
                       "* w_scale.astype(np.float64).mean() \\\n        * x_scale.astype(np.float64)[:, None]"),
    "input_not_quantized": ("    xq, xs = quantize_rows(x)\n    return q8_matmul(wq, ws, xq, xs)",
                            "    return (x.astype(np.float64) @ (wq.astype(np.float64) * ws[:, None]).T)"),
}


def _q8_mutant(name):
    src = inspect.getsource(Q8)
    old, new = Q8_MUTANTS[name]
    assert src.count(old) >= 1, f"mutation anchor for {name} not found"
    src = src.replace(old, new, 1)
    mod = types.ModuleType(f"q8_mutant_{name}")
    exec(compile(src, f"<q8 mutant {name}>", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(Q8_MUTANTS))
def test_q8_mutant_is_caught(name):
    mod = _q8_mutant(name)
    failures = []
    for pin in QP.ALL_PINS:
        try:
            with np.errstate(all="ignore"):
                pin(mod)
        except (AssertionError, FloatingPointError, ValueError, TypeError,
                OverflowError):
            failures.append(pin.__name__)
    assert failures, f"q8 mutant {name} passed every pin"
