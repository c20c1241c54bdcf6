"""Pins for the oracle's FP4 codebook and FP4 quantization (CPU only).

"bitsandbytes" page: the 4-bit training paragraph names FP4, "standard
floating-point 4-bit", beside NF4; the NF4 paragraph contrasts NF4 with FP4's
uniform floating-point spacing.  The reading (codes are the E2M1 bit
patterns, levels their values over 6) is checked here against things other
than the oracle's own formula: the E2M1 value table of the OCP Microscaling
format specification, exact rational rounding, and invariants.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle.nf4_oracle as O

# E2M1 (OCP Microscaling Formats specification v1.0, the FP4 element type):
# bit patterns 0b0000 .. 0b0111 encode these magnitudes; bit 3 is the sign.
E2M1_MAGNITUDES = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2),
                   Fraction(2), Fraction(3), Fraction(4), Fraction(6)]


def test_levels_are_the_e2m1_values_over_six():
    c = O.fp4_codebook()
    assert c.dtype == np.float32 and c.shape == (16,)
    for code in range(16):
        mag = E2M1_MAGNITUDES[code & 7] / 6
        want = np.float32(float(mag))          # k/12 never falls on a float32 midpoint
        if code >= 8:
            want = -want
        assert c[code] == want, code
    # +0 and -0, the extremes exactly +-1, the negative half the sign-flipped positive half
    assert c[0] == 0 and not np.signbit(c[0]) and c[8] == 0 and np.signbit(c[8])
    assert c[7] == 1.0 and c[15] == -1.0
    assert np.array_equal(c[8:].view(np.uint32), c[:8].view(np.uint32) | np.uint32(0x80000000))
    assert O.zero_code(c) == 0 and O.zero_code(O.codebook()) == 7


def _direct_code(n: np.float32, c: np.ndarray) -> int:
    """Nearest FP4 level by exact rationals: nearest magnitude, ties to the smaller, then the sign."""
    mags = [Fraction(float(c[i])) for i in range(8)]       # the float32 levels, exactly
    x = Fraction(float(n))
    ax = abs(x)
    best = min(range(8), key=lambda i: (abs(ax - mags[i]), i))
    return best + 8 if (x < 0 and best > 0) else best


def test_nearest_code_matches_exact_rounding_toward_zero_on_ties():
    c = O.fp4_codebook()
    rng = np.random.default_rng(11)
    pts = [np.float32(0.0), np.float32(-0.0), np.float32(1.0), np.float32(-1.0)]
    # every midpoint between adjacent magnitudes, both signs, and its float32 neighbours
    for i in range(7):
        mid = (float(c[i]) + float(c[i + 1])) / 2          # exact in float64
        for v in (mid, -mid):
            f = np.float32(v)
            pts += [f, np.nextafter(f, np.float32(2)), np.nextafter(f, np.float32(-2))]
    pts += list(rng.uniform(-1, 1, 4000).astype(np.float32))
    pts += list((rng.uniform(-1, 1, 500) * 1e-3).astype(np.float32))
    n = np.array(pts, np.float32)
    got = O.nearest_code(n, c)
    want = np.array([_direct_code(v, c) for v in n], np.uint8)
    assert np.array_equal(got, want)
    # exact midpoints that float32 can hold (1/8 between 1/12 and 1/6 is one) go toward zero
    assert O.nearest_code(np.array([0.125, -0.125], np.float32), c).tolist() == [1, 9]


@pytest.mark.parametrize("bs", [32, 64, 256])
def test_absmax_element_recovery_and_requantization_round_trip(bs):
    rng = np.random.default_rng(bs)
    w = (rng.standard_normal(bs * 37 + 5) * 0.02).astype(np.float32)
    qs = O.quantize(w, bs, double_quant_on=False, quant_type="fp4")
    codes, a = qs["codes"], qs["absmax"]
    # the element of largest magnitude in each block takes the level +-1 and comes back exactly
    blocks = np.pad(w, (0, -w.size % bs)).reshape(-1, bs)
    top = np.argmax(np.abs(blocks), axis=1)
    cb = np.pad(codes, (0, -codes.size % bs)).reshape(-1, bs)
    picked = cb[np.arange(cb.shape[0]), top]
    assert set(np.unique(picked).tolist()) <= {7, 15}
    wf = O.dequantize(qs, out="f32")
    wfb = np.pad(wf, (0, -wf.size % bs)).reshape(-1, bs)
    assert np.array_equal(np.abs(wfb[np.arange(wfb.shape[0]), top]), a)
    # quantizing the dequantized weight reproduces the codes
    again = O.quantize(wf, bs, double_quant_on=False, quant_type="fp4")
    assert np.array_equal(again["codes"], codes)


def test_zero_blocks_and_signed_zeros_take_code_zero():
    w = np.zeros(3 * 64, np.float32)
    w[64:128] = -0.0
    w[130] = 0.5
    w[131] = -0.0
    codes = O.quantize(w, 64, double_quant_on=False, quant_type="fp4")["codes"]
    assert np.all(codes[:128] == 0)                 # all-zero blocks, +0 and -0 alike
    assert codes[130] == 7 and codes[131] == 0      # the absmax element; a -0 beside it
    assert np.all(np.delete(codes[128:], [2, 3]) == 0)


def test_absmax_state_does_not_depend_on_the_codebook():
    rng = np.random.default_rng(3)
    w = (rng.standard_t(4, 64 * 600) * 0.02).astype(np.float32)
    a = O.quantize(w, 64, True, "nf4")
    b = O.quantize(w, 64, True, "fp4")
    for k in ("absmax", "absmax_q", "scale", "ahat"):
        assert np.array_equal(a[k], b[k]), k
    assert a["mean"] == b["mean"]
    assert not np.array_equal(a["codes"], b["codes"])
    # dequantization uses the FP4 table: level * a^ for every element
    wb = O.dequantize(b, out="f32")
    lv = O.fp4_codebook()[b["codes"]]
    ah = np.repeat(b["ahat"], 64)[: w.size]
    assert np.array_equal(wb, (lv * ah).astype(np.float32))
