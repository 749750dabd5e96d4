"""Streaming form of the parity metric, for comparisons too large to hold.

The metric (the tolerance is stated on max|err|/rms(o)): over every compared
element of a workload, max |got - ref| divided by the root mean square of
ref, in float64. `ParityMeter` accumulates the maximum absolute difference,
the sum of squares of the reference and the element count part by part, so
that a workload can be compared sequence by sequence; fed all of it at once
it gives exactly oracle.rel_max_err (tested on the CPU).
"""
from __future__ import annotations

import math

import numpy as np


# Summaries the tests report, printed at the end of the pytest run (the
# terminal summary shows them even when the tests' own output is captured).
REPORTED: list = []


def report(line: str) -> None:
    REPORTED.append(line)


class ParityMeter:
    def __init__(self, name: str = ""):
        self.name = name
        self.max_abs = 0.0
        self.sumsq = 0.0
        self.count = 0
        self.worst_part = 0.0      # the largest per-part rel_max_err seen
        self.worst_where = None
        self.nonfinite = 0

    def add(self, got, ref, where=None) -> float:
        """Add one part; returns that part's own max|err|/rms(ref)."""
        g = np.asarray(got, dtype=np.float64)
        r = np.asarray(ref, dtype=np.float64)
        if g.shape != r.shape:
            raise ValueError(f"shape mismatch {g.shape} vs {r.shape}")
        if g.size == 0:
            return 0.0
        self.nonfinite += int(np.count_nonzero(~np.isfinite(g)))
        d = float(np.max(np.abs(g - r)))
        if not math.isfinite(d):
            d = math.inf
        ss = float(np.sum(r * r))
        self.max_abs = max(self.max_abs, d)
        self.sumsq += ss
        self.count += g.size
        rms = math.sqrt(ss / g.size)
        part = d / rms if rms > 0 else d
        if part > self.worst_part or self.worst_where is None:
            self.worst_part, self.worst_where = part, where
        return part

    def value(self) -> float:
        if self.count == 0:
            return 0.0
        rms = math.sqrt(self.sumsq / self.count)
        if self.nonfinite:
            return math.inf
        return self.max_abs / rms if rms > 0 else self.max_abs

    def summary(self) -> str:
        return (f"{self.name}: max|err|/rms {self.value():.3e} over "
                f"{self.count} elements (worst part {self.worst_part:.3e} at "
                f"{self.worst_where})")
