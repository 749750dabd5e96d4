"""Pins of the INT8 oracle (page "RWKV-X Architecture", section "INT8
Quantization"), each a function of an oracle module M, so that the same pins
check the oracle and planted-mistake copies of it. They compare against what
the definition and arithmetic fix, computed independently of the oracle's
code: decimal rounding of exact values, exact rationals, closed forms on
exactly representable rows, brute-force integer sums and the quantization
error bound."""
from decimal import Decimal, ROUND_HALF_UP
from fractions import Fraction

import numpy as np

f32 = np.float32


def pin_roundf_is_half_away_from_zero(M):
    vals = [0.0, 0.5, 1.5, 2.5, -0.5, -1.5, -2.5, 126.5, -126.5, 3.25, -3.75]
    vals += [float(np.nextafter(f32(v), f32(0))) for v in (0.5, 1.5, -2.5, 99.5)]
    vals += [float(np.nextafter(f32(v), f32(10 * v))) for v in (0.5, -1.5, 7.5)]
    got = M.roundf(np.array(vals, np.float32))
    for v, g in zip(vals, got):
        want = Decimal(float(f32(v))).quantize(Decimal(1), rounding=ROUND_HALF_UP)
        assert float(g) == float(want), (v, g, want)


def pin_exact_integer_rows_are_reproduced(M):
    rng = np.random.default_rng(0)
    ints = rng.integers(-127, 128, size=(6, 40)).astype(np.float32)
    ints[:, 0] = 127.0 * np.where(np.arange(6) % 2, 1, -1)  # max |.| = 127
    s = np.float32(2.0) ** rng.integers(-20, 20, size=6).astype(np.float32)
    q, scale = M.quantize_rows(ints * s[:, None])
    assert np.array_equal(q.astype(np.float32), ints)
    assert np.array_equal(scale, s)


def pin_zero_and_single_entry_rows(M):
    x = np.zeros((3, 8), np.float32)
    x[1, 5] = -3.5
    x[2, 2] = 1e-30
    q, scale = M.quantize_rows(x)
    assert scale[0] == 0 and not q[0].any()
    assert q[1, 5] == -127 and np.count_nonzero(q[1]) == 1
    assert q[2, 2] == 127 and np.count_nonzero(q[2]) == 1


def pin_codes_match_exact_rational_rounding(M):
    """Away from ties, the code is the exact quotient x / scale (scale being
    the float32 value the oracle stores) rounded half away from zero."""
    rng = np.random.default_rng(1)
    x = rng.standard_normal((5, 33)).astype(np.float32)
    q, scale = M.quantize_rows(x)
    checked = 0
    for r in range(5):
        sc = Fraction(float(scale[r]))
        assert sc == Fraction(float(f32(np.max(np.abs(x[r]))) / f32(127)))
        for c in range(33):
            quot = Fraction(float(x[r, c])) / sc
            frac = abs(quot) - int(abs(quot))
            if abs(frac - Fraction(1, 2)) < Fraction(1, 1 << 18):
                continue        # the float32 quotient may round across .5
            mag = int(abs(quot)) + (1 if frac > Fraction(1, 2) else 0)
            assert int(q[r, c]) == (mag if quot >= 0 else -mag)
            checked += 1
    assert checked > 150


def pin_error_bound_and_range(M):
    rng = np.random.default_rng(2)
    x = (rng.standard_normal((8, 300)) * 10.0 ** rng.integers(-3, 4, (8, 1))
         ).astype(np.float32)
    q, scale = M.quantize_rows(x)
    assert np.abs(q.astype(np.int32)).max() == 127
    err = np.abs(x.astype(np.float64) - q.astype(np.float64) * scale[:, None])
    assert np.all(err <= scale[:, None].astype(np.float64) * (0.5 + 2.0 ** -20))
    # sign symmetry and power-of-two scale invariance
    qn, sn = M.quantize_rows(-x)
    assert np.array_equal(qn, -q) and np.array_equal(sn, scale)
    q4, s4 = M.quantize_rows(x * np.float32(4.0))
    assert np.array_equal(q4, q) and np.array_equal(s4, scale * np.float32(4.0))


def pin_matmul_brute_force_integers(M):
    rng = np.random.default_rng(3)
    wq = rng.integers(-127, 128, (5, 7)).astype(np.int8)
    xq = rng.integers(-127, 128, (3, 7)).astype(np.int8)
    ws = rng.random(5).astype(np.float32)
    xs = rng.random(3).astype(np.float32)
    y = M.q8_matmul(wq, ws, xq, xs)
    for b in range(3):
        for o in range(5):
            acc = sum(int(wq[o, i]) * int(xq[b, i]) for i in range(7))
            want = Fraction(acc) * Fraction(float(ws[o])) * Fraction(float(xs[b]))
            assert abs(Fraction(float(y[b, o])) - want) <= abs(want) * Fraction(1, 1 << 50)


def pin_quantized_linear_within_its_error_bound(M):
    rng = np.random.default_rng(4)
    w = rng.standard_normal((64, 256)).astype(np.float32)
    x = rng.standard_normal((6, 256)).astype(np.float32)
    y = M.q8_linear(w, x)
    exact = x.astype(np.float64) @ w.astype(np.float64).T
    _, ws = M.quantize_rows(w)
    _, xs = M.quantize_rows(x)
    dw = ws.astype(np.float64)[None, :, None] * 0.5 * (1 + 2.0 ** -20)
    dx = xs.astype(np.float64)[:, None, None] * 0.5 * (1 + 2.0 ** -20)
    aw = np.abs(w.astype(np.float64))[None, :, :]
    ax = np.abs(x.astype(np.float64))[:, None, :]
    bound = (dw * ax + aw * dx + dw * dx).sum(-1)
    assert np.all(np.abs(y - exact) <= bound)
    # and it is a useful approximation: about 1% of the output's rms
    assert np.max(np.abs(y - exact)) / np.sqrt(np.mean(exact ** 2)) < 0.05


def pin_input_rows_quantized_by_hand(M):
    """Hand-worked: w = [[0, 1]] gives codes [0, 127] at scale 1/127.
    x row [127, 0.4]: scale 1, codes [127, 0] (0.4 rounds to 0), so y = 0.
    x row [1, 0.4]: scale 1/127, codes [127, 51] (0.4 * 127 = 50.8), so
    y = 127 * 51 / 127^2 = 51/127. A per-tensor input scale would give 0."""
    w = np.array([[0.0, 1.0]], np.float32)
    x = np.array([[127.0, 0.4], [1.0, 0.4]], np.float32)
    y = M.q8_linear(w, x)
    assert y[0, 0] == 0.0
    s127 = Fraction(float(f32(1.0) / f32(127.0)))
    want = Fraction(127 * 51) * s127 * s127
    assert abs(Fraction(float(y[1, 0])) - want) <= want * Fraction(1, 1 << 50)
    assert abs(float(y[1, 0]) - 51.0 / 127.0) < 1e-6


ALL_PINS = [pin_input_rows_quantized_by_hand,
            pin_roundf_is_half_away_from_zero,
            pin_exact_integer_rows_are_reproduced,
            pin_zero_and_single_entry_rows,
            pin_codes_match_exact_rational_rounding,
            pin_error_bound_and_range,
            pin_matmul_brute_force_integers,
            pin_quantized_linear_within_its_error_bound]
