"""Plain, slow, obviously-correct CPU oracle for NF4 quantization and NF4 GEMMs.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py``; never by the product library.

Sources (cited by page title and passage; the pages print no code, no table
and no worked example):

* [zenbit] "Zenbit" (PyPI project page), section *What's inside*: the
  ``zenbit.nf4`` bullet (NF4 blockwise quantization with double quantization,
  QLoRA-style) and the ``zenbit.pallas_nf4`` bullet (fused NF4 dequant+matmul
  with the weight dequantized on chip, never materialised in HBM; fused
  backward that forms dL/dX only, dL/dW not computed for a frozen weight).
* [bnb-nf4] "bitsandbytes" (unfragile.ai artifact page), the paragraph on the
  NF4 data type: 16 levels from the inverse normal CDF, more levels near zero,
  weights mapped to levels through lookup tables after per-block statistics.
* [bnb-dq] same page, the paragraph on secondary (double) quantization:
  absmax per 64-weight block, the absmax values themselves quantized to 8 bits
  with their own meta-scales; scales are dequantized first, then used to
  dequantize the weights.
* [bnb-gemm] same page, the paragraph on quantized-weight GEMM kernels: weights
  dequantized on the fly, float32 multiply, float32 outputs.
* [bnb-lora] same page, the paragraph on 4-bit training with low-rank
  adapters: the 4-bit base weight stays frozen while small adapters train;
  the 4-bit data type is NF4 or FP4, "standard floating-point 4-bit".  The
  NF4 paragraph contrasts NF4 with FP4's uniform floating-point spacing, and
  the QuantState paragraph has the data type travel with the quantized state.

Readings taken where the pages are silent (each is listed, with the reason, in
the design notes of the repository):

* R1 codebook: QLoRA's asymmetric NF4 (Dettmers et al., 2023): 8 positive
  quantiles of N(0,1) at probabilities ``linspace(delta, 0.5, 9)[:-1]``, 7
  negative ones at ``linspace(delta, 0.5, 8)[:-1]``, plus 0, sorted, divided by
  the largest; ``delta = 0.9677083``; all in float64, one final rounding to
  float32.
* R2 normalisation is an IEEE float32 division ``n = fl(x / absmax)``; an
  all-zero block gets code 7 (the level 0.0) and absmax 0.
* R3 nearest level with ties to the lower index; two codes per byte, the even
  element in the low nibble; an odd element count leaves a zero high nibble.
* R4 double quantization: mu = the exact mean of all block absmax values
  rounded once to float32; a' = fl(a - mu); per group of 256 blocks
  s = fl(max|a'| / 127); q = clamp(round-half-even(fl(a'/s)), -127, 127);
  s = 0 and q = 0 for an all-zero group.
* R5 dequantization: a^ = fl(fl(q*s) + mu) (two roundings) with double
  quantization, else a^ = a; W^ = bf16_rne(fl(c[code] * a^)).
* R6 GEMMs: Y = X W^T and dX = dY W^ in float64 over bf16 operands; a result
  passes when |err| <= 1e-4 * (|X| |W^|^T) element by element.
* R7 adapter term: with an adapter of down projection A [r, K] and up
  projection B [N, r], the layer output is X W^T + (X A^T) B^T and its input
  gradient dY W^ + (dY B) A.  The fused calls take the bf16 down-projected
  activation U = X A^T (or V = dY B) as given and add U B^T (or V A) in the
  same accumulation; the bound adds the adapter product's magnitude term.
  The adapter's own products, with a scale s: U = s X A^T, V = s dY B and
  the gradients of the adapter weights dA = V^T X, dB = dY^T U (the
  gradient of the forward's U B^T term; U and V as the layer used them).
* R8 FP4 codebook: the standard 4-bit float E2M1 (one sign bit, two exponent
  bits with bias 1, one mantissa bit; magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6).
  A code is the format's own bit pattern (bit 3 the sign), its level the
  value divided by 6 (the largest) and rounded once to float32, so the table
  spans [-1, 1] like NF4's.  Quantization is the same nearest-level search
  with ties to the lower code, which in this encoding is toward zero on both
  sides; zero (and an all-zero block) takes code 0, the +0 level.

Arrays: a weight is a float32 numpy array (bf16 inputs are passed upcast to
float32, which is exact); bf16 outputs are returned as uint16 bit patterns.
"""
from __future__ import annotations

import math
import statistics

import numpy as np
from scipy.special import ndtri

__all__ = [
    "DELTA", "BLOCKSIZE", "DQ_GROUP", "GEMM_RTOL",
    "nf4_levels_f64", "codebook", "fp4_levels_f64", "fp4_codebook", "codebook_of", "zero_code",
    "QUANT_TYPES",
    "f32_to_bf16_bits", "bf16_bits_to_f32",
    "block_absmax", "normalize", "nearest_code", "encode_blocks", "pack_codes", "unpack_codes",
    "round_rational_to_f32", "exact_mean_f32",
    "double_quant", "dq_absmax", "dequantize_codes",
    "quantize", "dequantize", "nblocks_of", "ngroups_of",
    "matmul_fwd", "matmul_bwd_dx", "fwd_bound", "bwd_dx_bound", "gemm_violations", "ppf_stdlib",
    "matmul_fwd_lora", "matmul_bwd_dx_lora", "fwd_lora_bound", "bwd_dx_lora_bound",
    "adapter_down", "adapter_down_grad", "adapter_grad_down", "adapter_grad_up", "product_bound",
]

DELTA = 0.9677083          # R1: QLoRA's offset, the 7-digit literal
BLOCKSIZE = 64             # [bnb-dq]: absmax per 64-weight block
DQ_GROUP = 256             # R4: one fp32 meta-scale per 256 absmax values
GEMM_RTOL = 1e-4           # R6


# --------------------------------------------------------------------------- codebook (R1)

def nf4_levels_f64(ppf=ndtri):
    """The 16 NF4 levels in float64 (before the final float32 rounding).

    [bnb-nf4]: levels are quantiles of the standard normal (inverse CDF), with
    more of them near zero.  ``ppf`` is the inverse normal CDF to use; the
    tests build the table with three independent implementations.
    """
    p_pos = np.linspace(DELTA, 0.5, 9)[:-1]      # 8 probabilities above 1/2
    p_neg = np.linspace(DELTA, 0.5, 8)[:-1]      # 7 probabilities above 1/2
    positive = [float(ppf(float(p))) for p in p_pos]
    negative = [-float(ppf(float(p))) for p in p_neg]
    levels = sorted(positive + [0.0] + negative)
    top = max(levels)
    return [v / top for v in levels]


def codebook() -> np.ndarray:
    """The NF4 codebook: 16 ascending float32 levels, c[0] = -1, c[7] = 0, c[15] = 1."""
    return np.array(nf4_levels_f64(), dtype=np.float64).astype(np.float32)


def fp4_levels_f64():
    """The 16 FP4 levels in float64, indexed by code (R8).

    Code bits s e1 e0 m: an exponent field of 0 is subnormal, m * 2^-1; a
    field e >= 1 is 2^(e-1) * (1 + m/2).  The value is divided by the largest
    magnitude, 6.
    """
    out = []
    for code in range(16):
        s, e, m = code >> 3, (code >> 1) & 3, code & 1
        mag = m * 0.5 if e == 0 else 2.0 ** (e - 1) * (1 + m / 2)
        out.append((-mag if s else mag) / 6.0)
    return out


def fp4_codebook() -> np.ndarray:
    """The FP4 codebook by code: c[0] = +0, c[7] = 1, c[8] = -0, c[15] = -1 (R8)."""
    return np.array(fp4_levels_f64(), dtype=np.float64).astype(np.float32)


QUANT_TYPES = ("nf4", "fp4")


def codebook_of(quant_type: str = "nf4") -> np.ndarray:
    if quant_type == "nf4":
        return codebook()
    if quant_type == "fp4":
        return fp4_codebook()
    raise ValueError(f"unknown quant_type {quant_type!r}")


def zero_code(c: np.ndarray) -> int:
    """The code of the +0 level: what an all-zero block codes every element as (R2, R8)."""
    c = np.asarray(c, np.float32)
    return int(np.flatnonzero((c == 0) & ~np.signbit(c))[0])


# --------------------------------------------------------------------------- bf16 <-> fp32

def f32_to_bf16_bits(x) -> np.ndarray:
    """Round float32 values to bfloat16, nearest-even, returned as uint16 bits.

    bfloat16 keeps the top 16 bits of the float32 encoding; rounding adds half
    an ulp of the kept part (0x7FFF, plus 1 when the kept part is odd, so ties
    go to even) before truncating.  Finite inputs only (no overflow of the
    32-bit sum is then possible).
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u >> np.uint32(16)) & np.uint32(1)
    r += np.uint32(0x7FFF)
    r += u
    r >>= np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


# --------------------------------------------------------------------------- quantization

def nblocks_of(numel: int, blocksize: int = BLOCKSIZE) -> int:
    return -(-numel // blocksize)


def ngroups_of(nblocks: int, group: int = DQ_GROUP) -> int:
    return -(-nblocks // group)


def _blocks(x_flat: np.ndarray, blocksize: int) -> np.ndarray:
    """Row-major flat float32 array -> [nblocks, blocksize], the tail padded with 0."""
    nb = nblocks_of(x_flat.size, blocksize)
    pad = nb * blocksize - x_flat.size
    if pad:
        x_flat = np.concatenate([x_flat, np.zeros(pad, np.float32)])
    return x_flat.reshape(nb, blocksize)


def block_absmax(x_flat: np.ndarray, blocksize: int = BLOCKSIZE) -> np.ndarray:
    """a_b = max |x| over each block of ``blocksize`` consecutive elements ([bnb-dq]).

    Padding the last block with zeros leaves the maximum of the present
    elements unchanged.
    """
    x = np.asarray(x_flat, dtype=np.float32).ravel()
    return np.abs(_blocks(x, blocksize)).max(axis=1).astype(np.float32)


def normalize(x: np.ndarray, a: np.ndarray) -> np.ndarray:
    """n = fl32(x / a) element by element (R2).  ``a`` broadcasts per block."""
    with np.errstate(divide="ignore", invalid="ignore"):
        return (np.asarray(x, np.float32) / np.asarray(a, np.float32)).astype(np.float32)


def nearest_code(n: np.ndarray, c: np.ndarray | None = None, chunk: int = 1 << 16) -> np.ndarray:
    """argmin_i |n - c_i| with ties to the lower index (R3).

    The distances are taken in float64: a tie can only happen where n lies
    between two adjacent levels of similar magnitude, and there both
    differences are exact in float64; elsewhere the two distances differ by far
    more than float64 rounding.  ``np.argmin`` returns the first minimum,
    which is the lower index.
    """
    if c is None:
        c = codebook()
    c64 = np.asarray(c, np.float64)[None, :]
    n = np.asarray(n, np.float32).ravel()
    out = np.empty(n.size, dtype=np.uint8)
    dist = np.empty((min(chunk, n.size), c64.size), np.float64)
    for lo in range(0, n.size, chunk):
        seg = n[lo:lo + chunk].astype(np.float64)[:, None]
        d = dist[: seg.shape[0]]
        np.subtract(seg, c64, out=d)
        np.abs(d, out=d)
        out[lo:lo + chunk] = np.argmin(d, axis=1)
    return out


def encode_blocks(xb: np.ndarray, a: np.ndarray, c: np.ndarray | None = None) -> np.ndarray:
    """Codes of a [nb, bs] float32 block array given its per-block absmax ``a``.

    [bnb-nf4] / [zenbit]: divide by the block absmax, map to the nearest NF4
    level.  A block whose absmax is 0 codes every element as 7 (R2).
    """
    if c is None:
        c = codebook()
    xb = np.asarray(xb, np.float32)
    a = np.asarray(a, np.float32)
    n = normalize(xb, a[:, None])
    codes = nearest_code(n, c).reshape(xb.shape)
    codes[a == 0, :] = zero_code(c)
    return codes


def pack_codes(codes: np.ndarray) -> np.ndarray:
    """Two 4-bit codes per byte: element 2j in the low nibble, 2j+1 in the high (R3)."""
    codes = np.asarray(codes, np.uint8).ravel()
    if codes.size % 2:
        codes = np.concatenate([codes, np.zeros(1, np.uint8)])
    return (codes[0::2] | (codes[1::2] << 4)).astype(np.uint8)


def unpack_codes(packed: np.ndarray, numel: int) -> np.ndarray:
    packed = np.asarray(packed, np.uint8).ravel()
    out = np.empty(packed.size * 2, np.uint8)
    out[0::2] = packed & 0x0F
    out[1::2] = packed >> 4
    return out[:numel]


# --------------------------------------------------------------------------- double quantization (R4)

def round_rational_to_f32(num: int, den: int) -> np.float32:
    """Round the non-negative rational num/den to float32, nearest-even, in one step.

    Integer arithmetic only: find the scale 2**e at which the quotient has 24
    significant bits (or the subnormal lsb 2**-149), divide, and round on the
    remainder.
    """
    if num < 0 or den <= 0:
        raise ValueError("round_rational_to_f32 expects num >= 0, den > 0")
    if num == 0:
        return np.float32(0.0)
    e = num.bit_length() - den.bit_length() - 24
    while True:
        if e >= 0:
            d = den << e
            q, r = divmod(num, d)
        else:
            d = den
            q, r = divmod(num << -e, den)
        if q >= (1 << 24):
            e += 1
        elif q < (1 << 23) and e > -149:
            e -= 1
        else:
            break
    if e < -149:  # below the subnormal lsb: rescale to it
        e = -149
        d = den
        q, r = divmod(num << 149, den)
    if 2 * r > d or (2 * r == d and (q & 1)):
        q += 1
    val = math.ldexp(q, e)
    if val > float(np.finfo(np.float32).max):
        return np.float32(np.inf)
    return np.float32(val)


def exact_mean_f32(a: np.ndarray) -> np.float32:
    """mu = the mean of the float32 values ``a``, computed exactly, rounded once (R4).

    Every finite float32 is an integer multiple of 2**-149, so the sum is an
    exact integer count of 2**-149 units; the mean is that integer over
    len(a) * 2**149, rounded to float32.
    """
    a = np.asarray(a, np.float32).ravel()
    if a.size == 0:
        raise ValueError("mean of an empty set")
    if not np.all(np.isfinite(a)):
        raise ValueError("non-finite absmax")
    units = a.astype(np.float64) * (2.0 ** 149)          # exact: power-of-two scaling
    total = sum(int(v) for v in units.tolist())
    if total >= 0:
        return round_rational_to_f32(total, a.size << 149)
    return -round_rational_to_f32(-total, a.size << 149)


def double_quant(a: np.ndarray, mu: np.float32, group: int = DQ_GROUP):
    """Quantize the block absmax values to int8 with one float32 scale per group (R4).

    [bnb-dq]: the scaling factors themselves are quantized to 8 bits with
    meta-scales.  Returns (q int8 [nblocks], s float32 [ngroups]).
    """
    a = np.asarray(a, np.float32).ravel()
    nb = a.size
    ng = ngroups_of(nb, group)
    ac = (a - np.float32(mu)).astype(np.float32)                 # a' = fl(a - mu)
    pad = ng * group - nb
    acg = np.concatenate([ac, np.zeros(pad, np.float32)]).reshape(ng, group)
    m = np.abs(acg).max(axis=1).astype(np.float32)               # max |a'| per group
    s = (m / np.float32(127.0)).astype(np.float32)               # s = fl(m / 127)
    with np.errstate(divide="ignore", invalid="ignore"):
        r = (acg / s[:, None]).astype(np.float32)                # fl(a' / s)
    q = np.clip(np.rint(r), -127, 127)                           # round half to even
    q[m == 0, :] = 0
    return q.reshape(-1)[:nb].astype(np.int8), s


def dq_absmax(q: np.ndarray, s: np.ndarray, mu: np.float32, group: int = DQ_GROUP) -> np.ndarray:
    """a^ = fl(fl(q * s) + mu): scales are dequantized first ([bnb-dq], R5)."""
    q = np.asarray(q, np.int8).ravel()
    sb = np.repeat(np.asarray(s, np.float32), group)[: q.size]
    t = (q.astype(np.float32) * sb).astype(np.float32)
    return (t + np.float32(mu)).astype(np.float32)


def dequantize_codes(codes: np.ndarray, ahat: np.ndarray, blocksize: int = BLOCKSIZE,
                     out: str = "bf16", c: np.ndarray | None = None, chunk: int = 1 << 20) -> np.ndarray:
    """W^_e = bf16_rne(fl(c[code_e] * a^_b)) (R5); ``out='f32'`` returns fl(c * a^) unrounded."""
    if c is None:
        c = codebook()
    c = np.asarray(c, np.float32)
    codes = np.asarray(codes, np.uint8).ravel()
    ahat = np.asarray(ahat, np.float32)
    res = np.empty(codes.size, np.uint16 if out == "bf16" else np.float32)
    step = chunk - chunk % blocksize
    for lo in range(0, codes.size, step):
        cc = codes[lo:lo + step]
        ab = np.repeat(ahat[lo // blocksize: (lo + cc.size + blocksize - 1) // blocksize], blocksize)[: cc.size]
        prod = (c[cc] * ab).astype(np.float32)
        res[lo:lo + cc.size] = prod if out == "f32" else f32_to_bf16_bits(prod)
    return res


def quantize(w: np.ndarray, blocksize: int = BLOCKSIZE, double_quant_on: bool = True,
             quant_type: str = "nf4") -> dict:
    """Full 4-bit blockwise quantization of a float32 weight (row-major flattening).

    ``quant_type`` picks the codebook: "nf4" (R1) or "fp4" (R8).  Returns a dict
    with ``codes`` (uint8 per element), ``packed`` (uint8), ``absmax`` (float32
    per block), and with double quantization ``mean``, ``absmax_q`` (int8 per
    block), ``scale`` (float32 per group); plus ``ahat`` (the absmax the
    dequantizer uses).
    """
    w = np.asarray(w, np.float32).ravel()
    if not np.all(np.isfinite(w)):
        raise ValueError("non-finite weight: outside the method's domain")
    c = codebook_of(quant_type)
    a = block_absmax(w, blocksize)
    codes = encode_blocks(_blocks(w, blocksize), a, c).ravel()[: w.size]
    res = {"numel": w.size, "blocksize": blocksize, "codes": codes, "quant_type": quant_type,
           "packed": pack_codes(codes), "absmax": a, "double_quant": bool(double_quant_on)}
    if double_quant_on:
        mu = exact_mean_f32(a)
        q, s = double_quant(a, mu)
        res.update(mean=mu, absmax_q=q, scale=s, ahat=dq_absmax(q, s, mu))
    else:
        res["ahat"] = a
    return res


def dequantize(qs: dict, out: str = "bf16") -> np.ndarray:
    return dequantize_codes(qs["codes"], qs["ahat"], qs["blocksize"], out,
                            c=codebook_of(qs.get("quant_type", "nf4")))


# --------------------------------------------------------------------------- GEMMs (R6)

def matmul_fwd(x: np.ndarray, w_hat: np.ndarray) -> np.ndarray:
    """Y = X W^T in float64; X [M,K], W^ [N,K] ([zenbit] fused forward, [bnb-gemm])."""
    return np.asarray(x, np.float64) @ np.asarray(w_hat, np.float64).T


def matmul_bwd_dx(dy: np.ndarray, w_hat: np.ndarray) -> np.ndarray:
    """dX = dY W^ in float64; dY [M,N], W^ [N,K] ([zenbit] fused backward, dL/dX only)."""
    return np.asarray(dy, np.float64) @ np.asarray(w_hat, np.float64)


def fwd_bound(x: np.ndarray, w_hat: np.ndarray) -> np.ndarray:
    return GEMM_RTOL * (np.abs(np.asarray(x, np.float64)) @ np.abs(np.asarray(w_hat, np.float64)).T)


def bwd_dx_bound(dy: np.ndarray, w_hat: np.ndarray) -> np.ndarray:
    return GEMM_RTOL * (np.abs(np.asarray(dy, np.float64)) @ np.abs(np.asarray(w_hat, np.float64)))


def matmul_fwd_lora(x: np.ndarray, w_hat: np.ndarray, u: np.ndarray, b: np.ndarray) -> np.ndarray:
    """Y = X W^T + U B^T in float64; U [M,r], B [N,r] ([bnb-lora], R7)."""
    return matmul_fwd(x, w_hat) + np.asarray(u, np.float64) @ np.asarray(b, np.float64).T


def matmul_bwd_dx_lora(dy: np.ndarray, w_hat: np.ndarray, v: np.ndarray, a_t: np.ndarray) -> np.ndarray:
    """dX = dY W^ + V A in float64; V [M,r], A^T given as a_t [K,r] ([bnb-lora], R7)."""
    return matmul_bwd_dx(dy, w_hat) + np.asarray(v, np.float64) @ np.asarray(a_t, np.float64).T


def fwd_lora_bound(x, w_hat, u, b) -> np.ndarray:
    return fwd_bound(x, w_hat) + GEMM_RTOL * (np.abs(np.asarray(u, np.float64)) @ np.abs(np.asarray(b, np.float64)).T)


def bwd_dx_lora_bound(dy, w_hat, v, a_t) -> np.ndarray:
    return bwd_dx_bound(dy, w_hat) + GEMM_RTOL * (np.abs(np.asarray(v, np.float64)) @
                                                  np.abs(np.asarray(a_t, np.float64)).T)


def adapter_down(x: np.ndarray, a: np.ndarray, s: float) -> np.ndarray:
    """U = s X A^T in float64; X [M,K], A [r,K] ([bnb-lora], R7)."""
    return float(s) * (np.asarray(x, np.float64) @ np.asarray(a, np.float64).T)


def adapter_down_grad(dy: np.ndarray, b: np.ndarray, s: float) -> np.ndarray:
    """V = s dY B in float64; dY [M,N], B [N,r] ([bnb-lora], R7)."""
    return float(s) * (np.asarray(dy, np.float64) @ np.asarray(b, np.float64))


def adapter_grad_down(v: np.ndarray, x: np.ndarray) -> np.ndarray:
    """dA = V^T X in float64; V [M,r], X [M,K] -> [r,K] ([bnb-lora], R7)."""
    return np.asarray(v, np.float64).T @ np.asarray(x, np.float64)


def adapter_grad_up(dy: np.ndarray, u: np.ndarray) -> np.ndarray:
    """dB = dY^T U in float64; dY [M,N], U [M,r] -> [N,r] ([bnb-lora], R7)."""
    return np.asarray(dy, np.float64).T @ np.asarray(u, np.float64)


def product_bound(p: np.ndarray, q: np.ndarray, s: float = 1.0) -> np.ndarray:
    """1e-4 |s| (|P| |Q|) for a product s P Q of two matrices given as P [m,k], Q [k,n] (R6's bound)."""
    return GEMM_RTOL * abs(float(s)) * (np.abs(np.asarray(p, np.float64)) @ np.abs(np.asarray(q, np.float64)))


def gemm_violations(out: np.ndarray, ref: np.ndarray, bound: np.ndarray) -> int:
    """Number of elements with |out - ref| > bound (a zero bound demands equality)."""
    err = np.abs(np.asarray(out, np.float64) - ref)
    return int(np.count_nonzero(~(err <= bound)))


# --------------------------------------------------------------------------- alternative inverse CDFs

def ppf_stdlib(p: float) -> float:
    """Inverse normal CDF from Python's ``statistics.NormalDist`` (Wichura's AS241)."""
    return statistics.NormalDist().inv_cdf(p)
