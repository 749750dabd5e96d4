"""The parity metric itself, against hand-computed values (CPU only).

max |got - ref| / rms(ref) over every compared element, in float64: the
tolerance the workloads state is on max|err|/rms(o).
"""
import math

import numpy as np
import pytest

from oracle import rel_max_err
from tests.parity import ParityMeter


def test_rel_max_err_hand_computed():
    # |diff| = (0, 0, 2); rms(ref) = sqrt((1 + 4 + 25) / 3) = sqrt(10)
    got = np.array([1.0, 2.0, 3.0])
    ref = np.array([1.0, 2.0, 5.0])
    assert rel_max_err(got, ref) == pytest.approx(2.0 / math.sqrt(10.0),
                                                  rel=1e-15)
    # the sign of the difference does not matter
    assert rel_max_err(ref, got) == pytest.approx(
        2.0 / math.sqrt((1 + 4 + 9) / 3.0), rel=1e-15)
    # 2-D arrays: every element counts once; rms over all of them
    g2 = np.array([[0.0, 1.0], [1.0, 0.5]])
    r2 = np.array([[0.0, 1.0], [-1.0, 0.0]])
    # |diff| max = 2; rms = sqrt(2 / 4)
    assert rel_max_err(g2, r2) == pytest.approx(2.0 / math.sqrt(0.5),
                                                rel=1e-15)


def test_rel_max_err_special_cases():
    assert rel_max_err(np.zeros(0), np.zeros(0)) == 0.0
    # a zero reference falls back to the absolute difference
    assert rel_max_err(np.array([0.5, -0.25]), np.zeros(2)) == 0.5
    # an explicit scale replaces ref in the denominator only
    assert rel_max_err(np.array([1.0, 1.0]), np.array([1.0, 0.0]),
                       scale=np.array([2.0, 2.0])) == 0.5
    # identical arrays give exactly zero
    x = np.random.default_rng(0).standard_normal(100)
    assert rel_max_err(x, x) == 0.0
    # a NaN in the result is never a pass
    assert not (rel_max_err(np.array([np.nan, 1.0]), np.ones(2)) < 1.0)


def test_meter_parts_equal_whole():
    rng = np.random.default_rng(1)
    ref = rng.standard_normal((7, 5, 3))
    got = ref + rng.standard_normal(ref.shape) * 1e-3
    m = ParityMeter("x")
    for i in range(7):
        m.add(got[i], ref[i], where=i)
    assert m.value() == pytest.approx(rel_max_err(got, ref), rel=1e-13)
    assert m.count == ref.size
    # the worst part is a part's own metric, never below the whole's max diff
    # over that part's rms
    i = m.worst_where
    assert m.worst_part == pytest.approx(rel_max_err(got[i], ref[i]),
                                         rel=1e-13)


def test_meter_nonfinite_fails():
    m = ParityMeter()
    m.add(np.array([1.0, np.inf]), np.array([1.0, 1.0]))
    assert m.value() == math.inf
    m2 = ParityMeter()
    m2.add(np.array([np.nan]), np.array([1.0]))
    assert not (m2.value() < 1.0)
    with pytest.raises(ValueError):
        m2.add(np.zeros(2), np.zeros(3))
