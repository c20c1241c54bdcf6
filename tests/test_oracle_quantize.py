"""Pins for the oracle's NF4 blockwise quantizer (absmax, nearest level, packing).

Pinned against exact rational arithmetic, brute force and invariants; the
pages print no worked example.  Method passages: "Zenbit" page, *What's inside*,
``zenbit.nf4`` bullet; "bitsandbytes" page, NF4 data-type and double
quantization paragraphs (absmax per 64-weight block).
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle as O
from tests._exact import exact_argmin_code


def _all_bf16_in_unit_interval():
    u = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    v = (u.astype(np.uint32) << 16).view(np.float32)
    v = v[np.isfinite(v) & (np.abs(v) <= 1.0)]
    return np.unique(v)


def _fp32_ulps_around(x: float, k: int):
    x = np.float32(x)
    out = [x]
    lo = hi = x
    for _ in range(k):
        lo = np.nextafter(lo, np.float32(-np.inf))
        hi = np.nextafter(hi, np.float32(np.inf))
        out += [lo, hi]
    return np.array(out, np.float32)


def _midpoints():
    c = O.codebook()
    return [(Fraction(float(c[i])) + Fraction(float(c[i + 1]))) / 2 for i in range(15)]


def test_nearest_level_bruteforce_exhaustive_bf16_and_threshold_neighbourhoods():
    c = O.codebook()
    pts = [_all_bf16_in_unit_interval()]
    for m in _midpoints():
        pts.append(_fp32_ulps_around(float(m), 64))
    n = np.concatenate(pts)
    got = O.nearest_code(n, c)
    want = np.array([exact_argmin_code(v, c) for v in n], np.uint8)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, f"{bad.size} mismatches, first n={n[bad[0]]!r}"
    assert n.size > 30000


def test_exact_midpoints_go_to_the_lower_index():
    c = O.codebook()
    exact = []
    for i, m in enumerate(_midpoints()):
        f = np.float32(float(m))
        if Fraction(float(f)) == m:
            exact.append(i)
            assert O.nearest_code(np.array([f]), c)[0] == i
            # one ulp above the tie goes up
            assert O.nearest_code(np.array([np.nextafter(f, np.float32(2))]), c)[0] == i + 1
    # five of the fifteen midpoints are float32 numbers: c2|c3, c3|c4, c6|c7, c7|c8, c10|c11
    assert exact == [2, 3, 6, 7, 10]


def test_pack_hand_example():
    # codes [0, 15, 7, 8]: byte 0 = 0 | 15 << 4, byte 1 = 7 | 8 << 4
    assert O.pack_codes(np.array([0, 15, 7, 8], np.uint8)).tolist() == [0xF0, 0x87]
    assert O.pack_codes(np.array([1, 2, 3], np.uint8)).tolist() == [0x21, 0x03]


def test_pack_unpack_roundtrip():
    rng = np.random.default_rng(5)
    for numel in (1, 2, 63, 64, 65, 1001):
        codes = rng.integers(0, 16, numel).astype(np.uint8)
        packed = O.pack_codes(codes)
        assert packed.size == (numel + 1) // 2
        assert np.array_equal(O.unpack_codes(packed, numel), codes)


def test_zero_block_codes_seven():
    w = np.zeros(128, np.float32)
    w[64:] = np.linspace(-1, 1, 64, dtype=np.float32)
    q = O.quantize(w, double_quant_on=False)
    assert q["absmax"][0] == 0.0
    assert np.all(q["codes"][:64] == 7)
    assert np.all(O.dequantize(q)[:64] == 0)


def test_elementwise_bruteforce_small():
    """Each code equals the exact nearest level of fl32(x / absmax)."""
    rng = np.random.default_rng(11)
    w = (rng.standard_normal(64 * 40) * 0.02).astype(np.float32)
    w[64:128] = rng.standard_t(4, 64).astype(np.float32)            # heavy tail
    w[128:192] = np.float32(1e-40) * rng.integers(-5, 6, 64)        # subnormal block
    w[192:256] = np.float32(3e38) * rng.uniform(-1, 1, 64).astype(np.float32)  # near overflow
    q = O.quantize(w, double_quant_on=False)
    c = O.codebook()
    for b in range(w.size // 64):
        blk = w[64 * b: 64 * b + 64]
        a = max(abs(float(v)) for v in blk)
        assert q["absmax"][b] == np.float32(a)
        for i, x in enumerate(blk):
            if a == 0:
                want = 7
            else:
                n = np.float32(x) / np.float32(a)          # the IEEE float32 quotient
                want = exact_argmin_code(n, c)
            assert q["codes"][64 * b + i] == want, (b, i)


def test_absmax_element_recovery():
    rng = np.random.default_rng(3)
    w = (rng.standard_normal(64 * 500) * 0.02).astype(np.float32)
    q = O.quantize(w, double_quant_on=False)
    wh = O.bf16_bits_to_f32(O.dequantize(q))
    for b in range(500):
        blk = w[64 * b: 64 * b + 64]
        i = int(np.argmax(np.abs(blk)))
        code = q["codes"][64 * b + i]
        assert code == (15 if blk[i] > 0 else 0)
        want = O.bf16_bits_to_f32(O.f32_to_bf16_bits(np.array([abs(blk[i])], np.float32)))[0]
        assert wh[64 * b + i] == np.copysign(want, blk[i])


def test_partial_block_and_odd_numel():
    rng = np.random.default_rng(8)
    w = rng.standard_normal(101).astype(np.float32)
    q = O.quantize(w, double_quant_on=True)
    assert q["absmax"].size == 2 and q["packed"].size == 51
    assert q["absmax"][1] == np.abs(w[64:]).max()
    assert q["packed"][-1] >> 4 == 0
    assert q["scale"].size == 1


@pytest.mark.parametrize("dq", [False, True])
@pytest.mark.parametrize("dist", ["normal", "student_t"])
def test_requantizing_dequantized_weights_reproduces_codes(dq, dist):
    rng = np.random.default_rng(21)
    if dist == "normal":
        w = (rng.standard_normal(1 << 16) * 0.02).astype(np.float32)
    else:
        w = (rng.standard_t(4, 1 << 20) * 0.02).astype(np.float32)
    q = O.quantize(w, double_quant_on=dq)
    wh = O.bf16_bits_to_f32(O.dequantize(q))
    q2 = O.quantize(wh, double_quant_on=False)
    ok_blocks = (q["ahat"] > 0) & (q["ahat"] >= np.float32(2.0 ** -100))
    mask = np.repeat(ok_blocks, 64)[: w.size]
    assert ok_blocks.mean() > 0.99
    assert np.array_equal(q2["codes"][mask], q["codes"][mask])


def test_nonfinite_input_is_refused():
    w = np.zeros(64, np.float32)
    w[3] = np.inf
    with pytest.raises(ValueError):
        O.quantize(w)
    w[3] = np.nan
    with pytest.raises(ValueError):
        O.quantize(w)


def test_bf16_rounding_matches_torch():
    """The oracle's bf16 rounding against torch's float->bfloat16 conversion (RNE)."""
    rng = np.random.default_rng(2)
    x = np.concatenate([
        rng.standard_normal(100000).astype(np.float32),
        (rng.standard_normal(1000) * 1e-39).astype(np.float32),                # subnormal
        ((np.arange(2000, dtype=np.uint32) << 15) | 0x3F800000).view(np.float32),  # exact ties
        np.array([0.0, -0.0, 1.0, -1.0, 3.3895314e38], np.float32),
    ])
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(O.f32_to_bf16_bits(x), want)
    assert np.array_equal(O.bf16_bits_to_f32(want), torch.from_numpy(want.view(np.int16)).view(torch.bfloat16).float().numpy())


def test_dequantized_block_values_lie_in_the_block_lut():
    rng = np.random.default_rng(4)
    w = (rng.standard_normal(64 * 300) * 0.02).astype(np.float32)
    q = O.quantize(w, double_quant_on=True)
    wh = O.dequantize(q)
    c = O.codebook()
    for b in range(300):
        lut = O.f32_to_bf16_bits((c * q["ahat"][b]).astype(np.float32))
        vals = set(wh[64 * b: 64 * b + 64].tolist())
        assert len(vals) <= 16 and vals <= set(lut.tolist())


# ------------------------------------------------------------------ other block sizes
# The absmax block is 64 weights on the pages ("bitsandbytes" page, double
# quantization paragraph); the same definition with 32, 128 or 256 weights per
# block is pinned the same way: exact absmax, exact nearest level of the IEEE
# quotient, and the relation between the absmax of neighbouring block sizes.

@pytest.mark.parametrize("bs", [32, 128, 256])
def test_elementwise_bruteforce_other_block_sizes(bs):
    rng = np.random.default_rng(40 + bs)
    n = bs * 12 + bs // 2 + 3                                             # partial last block
    w = (rng.standard_normal(n) * 0.02).astype(np.float32)
    w[bs:2 * bs] = rng.standard_t(4, bs).astype(np.float32)
    w[2 * bs:3 * bs] = np.float32(1e-40) * rng.integers(-5, 6, bs)
    w[3 * bs:4 * bs] = 0.0
    q = O.quantize(w, blocksize=bs, double_quant_on=False)
    c = O.codebook()
    nb = -(-n // bs)
    assert q["absmax"].size == nb and q["packed"].size == (n + 1) // 2
    for b in range(nb):
        blk = w[bs * b: bs * b + bs]
        a = max(abs(float(v)) for v in blk)
        assert q["absmax"][b] == np.float32(a)
        for i, x in enumerate(blk):
            want = 7 if a == 0 else exact_argmin_code(np.float32(x) / np.float32(a), c)
            assert q["codes"][bs * b + i] == want, (bs, b, i)


@pytest.mark.parametrize("bs", [32, 64, 128])
def test_absmax_of_doubled_block_size(bs):
    rng = np.random.default_rng(7)
    w = (rng.standard_t(4, bs * 2 * 100 + 37) * 0.02).astype(np.float32)
    a1 = O.quantize(w, blocksize=bs, double_quant_on=False)["absmax"]
    a2 = O.quantize(w, blocksize=2 * bs, double_quant_on=False)["absmax"]
    pairs = np.maximum(a1[0::2][: a2.size], np.append(a1[1::2], np.float32(0))[: a2.size])
    assert np.array_equal(a2, pairs)


@pytest.mark.parametrize("bs", [32, 256])
def test_double_quant_and_round_trip_other_block_sizes(bs):
    rng = np.random.default_rng(50 + bs)
    w = (rng.standard_normal(bs * 256 * 3 + bs * 5) * 0.02).astype(np.float32)
    q = O.quantize(w, blocksize=bs, double_quant_on=True)
    nb = -(-w.size // bs)
    assert q["absmax_q"].size == nb and q["scale"].size == -(-nb // 256)
    mean = sum(Fraction(float(a)) for a in q["absmax"]) / nb
    assert abs(Fraction(float(q["mean"])) - mean) <= abs(mean) * Fraction(1, 2 ** 24)
    err = np.abs(q["ahat"].astype(np.float64) - q["absmax"])
    s_per_block = np.repeat(q["scale"], 256)[:nb].astype(np.float64)
    assert np.all(err <= s_per_block / 2 + 4 * np.spacing(np.abs(q["absmax"]).astype(np.float32)))
    wh = O.bf16_bits_to_f32(O.dequantize(q))
    q2 = O.quantize(wh, blocksize=bs, double_quant_on=False)
    ok = np.repeat(q["ahat"] > 0, bs)[: w.size]
    assert np.array_equal(q2["codes"][ok], q["codes"][ok])
