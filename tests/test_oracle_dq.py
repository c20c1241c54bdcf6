"""Pins for the oracle's double quantization (exact mean, int8 absmax, meta-scales).

Method passage: "bitsandbytes" page, double quantization paragraph (absmax per
64-weight block quantized to 8 bits with its own meta-scales; scales
dequantized first, then the weights).  The centring on the global mean, int8
round-half-even and one fp32 scale per 256 values are the stated reading.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle as O
from tests._exact import nearest_f32


def _rand_rationals(rng, n):
    out = []
    for _ in range(n):
        num = int(rng.integers(1, 1 << 62)) << int(rng.integers(0, 200))
        den = int(rng.integers(1, 1 << 62)) << int(rng.integers(0, 360))
        out.append((num, den))
    return out


def test_round_rational_matches_neighbour_search():
    rng = np.random.default_rng(0)
    for num, den in _rand_rationals(rng, 3000):
        fr = Fraction(num, den)
        if fr > Fraction(float(np.finfo(np.float32).max)):
            continue
        assert O.round_rational_to_f32(num, den) == nearest_f32(fr), (num, den)


def test_round_rational_ties_go_to_even():
    # exact midpoints between neighbouring float32 values, normal and subnormal
    for base in (1.0, 1.5, 2.0 ** -126, 2.0 ** -140, 12345.0, 2.0 ** 100):
        a = np.float32(base)
        b = np.nextafter(a, np.float32(np.inf))
        mid = (Fraction(float(a)) + Fraction(float(b))) / 2
        got = O.round_rational_to_f32(mid.numerator, mid.denominator)
        even = a if int(a.view(np.uint32)) % 2 == 0 else b
        assert got == even


def _fraction_mean_f32(a):
    s = sum((Fraction(float(v)) for v in a), Fraction(0))
    return nearest_f32(s / len(a))


@pytest.mark.parametrize("case", ["normal", "subnormal", "wide", "ties"])
def test_exact_mean_against_fractions(case):
    rng = np.random.default_rng({"normal": 1, "subnormal": 2, "wide": 3, "ties": 4}[case])
    if case == "normal":
        a = np.abs(rng.standard_normal(777) * 0.05).astype(np.float32)
    elif case == "subnormal":
        a = (np.abs(rng.standard_normal(333)) * 1e-40).astype(np.float32)
    elif case == "wide":
        a = np.abs(rng.standard_normal(500) * 10.0 ** rng.integers(-30, 30, 500)).astype(np.float32)
    else:
        # sums that land exactly halfway between float32 neighbours
        a = np.array([1.0, np.nextafter(np.float32(1.0), np.float32(2.0))], np.float32)
    assert O.exact_mean_f32(a) == _fraction_mean_f32(a)


def test_exact_mean_is_permutation_invariant():
    rng = np.random.default_rng(9)
    a = np.abs(rng.standard_t(4, 100000) * 0.02).astype(np.float32)
    mu = O.exact_mean_f32(a)
    for _ in range(3):
        assert O.exact_mean_f32(rng.permutation(a)) == mu
    assert O.exact_mean_f32(a[:2000]) == _fraction_mean_f32(a[:2000])


def test_all_equal_absmax_gives_zero_int8_and_exact_recovery():
    a = np.full(600, np.float32(0.0371), np.float32)
    mu = O.exact_mean_f32(a)
    assert mu == a[0]
    q, s = O.double_quant(a, mu)
    assert np.all(q == 0) and np.all(s == 0)
    assert np.array_equal(O.dq_absmax(q, s, mu), a)


def test_one_outlier_per_group_attains_127():
    rng = np.random.default_rng(1)
    a = np.abs(rng.standard_normal(1024) * 0.01).astype(np.float32) + np.float32(0.05)
    for g in range(4):
        a[256 * g + 17] = np.float32(3.0)
    mu = O.exact_mean_f32(a)
    q, s = O.double_quant(a, mu)
    for g in range(4):
        assert q[256 * g + 17] == 127
        assert s[g] == np.float32(np.float32(3.0) - mu) / np.float32(127)


def test_int8_rounding_is_half_even():
    # mu = 0 so a' = a; max |a'| = 127 gives s = 1 and a'/s = a' exactly
    a = np.array([127.0, 2.5, 3.5, -2.5, -3.5, 0.5, 1.5, 126.5], np.float32)
    q, s = O.double_quant(a, np.float32(0.0))
    assert s[0] == 1.0
    assert q.tolist() == [127, 2, 4, -2, -4, 0, 2, 126]


def test_dq_error_bound():
    rng = np.random.default_rng(7)
    a = np.abs(rng.standard_t(4, 256 * 64) * 0.02).astype(np.float32)
    mu = O.exact_mean_f32(a)
    q, s = O.double_quant(a, mu)
    ah = O.dq_absmax(q, s, mu)
    sb = np.repeat(s, 256).astype(np.float64)
    ulp = np.spacing(np.maximum(np.abs(a), np.abs(ah))).astype(np.float64)
    err = np.abs(ah.astype(np.float64) - a.astype(np.float64))
    assert np.all(err <= sb / 2 + 3 * ulp)
    assert np.all(np.abs(q.astype(int)) <= 127)


def test_dq_absmax_is_two_roundings_not_fma():
    """a^ = RNE(RNE(q*s) + mu), computed here with exact rationals."""
    rng = np.random.default_rng(12)
    a = np.abs(rng.standard_normal(256 * 40) * 0.03).astype(np.float32)
    mu = O.exact_mean_f32(a)
    q, s = O.double_quant(a, mu)
    ah = O.dq_absmax(q, s, mu)
    differs_from_fma = 0
    for b in range(0, a.size, 7):
        prod = nearest_f32(Fraction(int(q[b])) * Fraction(float(s[b // 256])))
        two = nearest_f32(Fraction(float(prod)) + Fraction(float(mu)))
        fma = nearest_f32(Fraction(int(q[b])) * Fraction(float(s[b // 256])) + Fraction(float(mu)))
        assert ah[b] == two
        differs_from_fma += int(two != fma)
    assert differs_from_fma > 0  # the sample does distinguish the two readings


def test_quantize_without_dq_keeps_fp32_absmax():
    rng = np.random.default_rng(13)
    w = rng.standard_normal(64 * 10).astype(np.float32)
    q = O.quantize(w, double_quant_on=False)
    assert np.array_equal(q["ahat"], q["absmax"])
    assert "absmax_q" not in q


def test_mean_centring_uses_every_block():
    """mu is the mean over all blocks of the tensor, not per group."""
    a = np.concatenate([np.full(256, 1.0, np.float32), np.full(256, 3.0, np.float32)])
    mu = O.exact_mean_f32(a)
    assert mu == 2.0
    q, s = O.double_quant(a, mu)
    assert np.all(q[:256] == -127) and np.all(q[256:] == 127)
    assert np.array_equal(O.dq_absmax(q, s, mu), a)
