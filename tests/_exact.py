"""Exact-arithmetic helpers used by the oracle pins (pure Python, no oracle code).

They re-derive values from first principles (Python fractions and float32
neighbour search) so that the oracle's own arithmetic is checked against a
different route, not against itself.
"""
from fractions import Fraction

import numpy as np


def f32_neighbours(x: np.float32):
    x = np.float32(x)
    return [np.nextafter(x, np.float32(-np.inf)), x, np.nextafter(x, np.float32(np.inf))]


def nearest_f32(fr: Fraction) -> np.float32:
    """The float32 nearest to the rational ``fr``, ties to an even significand.

    Starts from numpy's float64 -> float32 conversion of ``float(fr)`` (which
    may be off by one ulp through double rounding) and picks the exact nearest
    of that value and its two neighbours.
    """
    guess = np.float32(float(fr))
    best = None
    for cand in f32_neighbours(guess) + f32_neighbours(np.nextafter(guess, np.float32(np.inf)))[1:] \
            + f32_neighbours(np.nextafter(guess, np.float32(-np.inf)))[:1]:
        if not np.isfinite(cand):
            continue
        d = abs(Fraction(float(cand)) - fr)
        if best is None or d < best[0]:
            best = (d, cand)
        elif d == best[0]:
            # tie: keep the one with an even last significand bit
            if int(np.float32(cand).view(np.uint32)) & 1 == 0:
                best = (d, cand)
    return np.float32(best[1])


def exact_argmin_code(n: np.float32, levels) -> int:
    """argmin_i |n - c_i| in exact rationals, first (lowest) index on ties."""
    fn = Fraction(float(n))
    best_i, best_d = None, None
    for i, c in enumerate(levels):
        d = abs(fn - Fraction(float(c)))
        if best_d is None or d < best_d:
            best_i, best_d = i, d
    return best_i
