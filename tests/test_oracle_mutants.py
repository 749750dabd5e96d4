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

import oracle.wkv7_oracle as ORC
from tests import oracle_pins as P

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
