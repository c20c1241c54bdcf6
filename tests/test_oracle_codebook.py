"""Pins for the oracle's NF4 codebook.

The pages state only that the 16 NF4 levels come from the inverse normal CDF
with more levels near zero ("bitsandbytes" page, NF4 data-type paragraph); the
construction (QLoRA's asymmetric 8/7 split with offset 0.9677083) is a reading.
These tests pin the oracle's table to the mathematics, not to itself:
three independent inverse-CDF implementations, the forward CDF, and the
structural invariants.
"""
from fractions import Fraction

import mpmath
import numpy as np
import pytest
from scipy.special import ndtr

import oracle as O
from tests._exact import nearest_f32


def _table_from_mpmath():
    """The same construction at 60 significant digits, exact probabilities."""
    mpmath.mp.dps = 60
    delta = mpmath.mpf(O.DELTA)  # exact binary value of the float64 literal
    half = mpmath.mpf(1) / 2

    def ppf(p):
        return mpmath.sqrt(2) * mpmath.erfinv(2 * p - 1)

    pos = [ppf(delta + j * (half - delta) / 8) for j in range(8)]
    neg = [-ppf(delta + j * (half - delta) / 7) for j in range(7)]
    levels = sorted(pos + [mpmath.mpf(0)] + neg)
    top = max(levels)
    out = []
    for v in levels:
        r = v / top
        # 55 significant digits: far finer than the closest level's distance
        # to a float32 rounding boundary (about 1e-10 relative)
        out.append(nearest_f32(Fraction(mpmath.nstr(r, 55, min_fixed=-1, max_fixed=1))))
    return np.array(out, dtype=np.float32)


def test_three_inverse_cdfs_agree_bit_for_bit():
    scipy_tab = O.codebook()
    stdlib_tab = np.array(O.nf4_levels_f64(O.ppf_stdlib), np.float64).astype(np.float32)
    mp_tab = _table_from_mpmath()
    assert scipy_tab.view(np.uint32).tolist() == stdlib_tab.view(np.uint32).tolist()
    assert scipy_tab.view(np.uint32).tolist() == mp_tab.view(np.uint32).tolist()


def test_codebook_invariants():
    c = O.codebook()
    assert c.dtype == np.float32 and c.shape == (16,)
    assert np.all(np.diff(c.astype(np.float64)) > 0)
    assert c[0] == -1.0 and c[7] == 0.0 and c[15] == 1.0
    assert np.count_nonzero(c < 0) == 7 and np.count_nonzero(c > 0) == 8


def test_delta_is_the_qlora_offset():
    # QLoRA's offset is the mean of 1 - 1/(2*15) and 1 - 1/(2*16), truncated to 7 digits.
    exact = (Fraction(29, 30) + Fraction(31, 32)) / 2
    assert exact == Fraction(929, 960)
    assert abs(Fraction(O.DELTA) - exact) < Fraction(1, 10 ** 7)


def test_levels_are_normal_quantiles():
    """Forward CDF check: Phi(c_i * Phi^-1(delta)) lands on the probability grid."""
    c = O.codebook().astype(np.float64)
    top = float(mpmath.sqrt(2) * mpmath.erfinv(2 * mpmath.mpf(O.DELTA) - 1))
    pos_grid = sorted(np.linspace(O.DELTA, 0.5, 9)[:-1])
    neg_grid = sorted(np.linspace(O.DELTA, 0.5, 8)[:-1])
    got_pos = ndtr(c[8:] * top)
    got_neg = ndtr(-c[:7] * top)
    assert np.allclose(np.sort(got_pos), pos_grid, rtol=0, atol=2e-7)
    assert np.allclose(np.sort(got_neg), neg_grid, rtol=0, atol=2e-7)


def test_more_levels_near_zero():
    c = O.codebook().astype(np.float64)
    gaps_neg = np.diff(c[:8])      # from -1 up to 0
    gaps_pos = np.diff(c[7:])      # from 0 up to +1
    assert np.all(np.diff(gaps_neg) < 0)   # gaps shrink approaching 0 from below
    assert np.all(np.diff(gaps_pos) > 0)   # and grow leaving 0 upwards


@pytest.mark.parametrize("wrong", ["fp32_intermediates", "symmetric"])
def test_plausible_mistakes_change_the_table(wrong):
    """The pins above distinguish the reading from two easy mistakes."""
    c = O.codebook()
    if wrong == "fp32_intermediates":
        from scipy.special import ndtri
        p_pos = np.linspace(np.float32(O.DELTA), np.float32(0.5), 9, dtype=np.float32)[:-1]
        p_neg = np.linspace(np.float32(O.DELTA), np.float32(0.5), 8, dtype=np.float32)[:-1]
        v = sorted(list(ndtri(p_pos).astype(np.float32)) + [np.float32(0)]
                   + list((-ndtri(p_neg)).astype(np.float32)))
        alt = (np.array(v, np.float32) / np.float32(max(v))).astype(np.float32)
    else:
        from scipy.special import ndtri
        p = np.linspace(O.DELTA, 0.5, 9)[:-1]
        v = sorted(list(ndtri(p)) + [0.0] + list(-ndtri(p[:7])))
        alt = (np.array(v) / max(v)).astype(np.float32)
    assert alt.view(np.uint32).tolist() != c.view(np.uint32).tolist()
