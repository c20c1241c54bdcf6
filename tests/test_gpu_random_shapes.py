"""GPU parity on seeded random shapes across every GEMM kernel's dispatch range.

"Zenbit" page, zenbit.pallas_nf4 bullet: the fused forward Y = X W^T and the
fused backward dX = dY W^.  Shapes are drawn (fixed seed) so that the cases
fall on all sides of the dispatch rules -- M from 1 to 1,200 (the small-M
kernel, its 16-row grid rows, the 256x256 kernel), N with and without
N % 8 == 0 (the backward's transposing and generic kernels), N up to 6,000 and not a
multiple of 16 or 64, K any multiple of 64 up to 1,280 (odd chunk and
double-step counts) -- with the block size, double quantization, codebook and
output dtype drawn as well.  Every element is compared with the oracle's
float64 products at 1e-4 * (|A| |B|); bf16 outputs must be the one rounding of
the fp32 results.
"""
import numpy as np
import pytest
import torch

import oracle as O
import synth
from tests._gpu import assert_gemm_within_bound, bf16_bits, dev, lib, note

pytestmark = pytest.mark.gpu


def _cases(n=32, seed=20261203):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        M = int(rng.choice([int(rng.integers(1, 17)), int(rng.integers(17, 260)), int(rng.integers(260, 1201))]))
        N = int(rng.integers(1, 6001))
        if i % 3 == 0:
            N = max(8, N - N % 8)             # the backward's 16-byte dY rows
        K = 64 * int(rng.integers(1, 21))
        bs = int(rng.choice([32, 64, 64, 128, 256]))
        dq = bool(rng.integers(0, 2))
        qt = "fp4" if rng.random() < 0.25 else "nf4"
        out.append((M, N, K, bs, dq, qt, 5000 + i))
    return out


@pytest.mark.parametrize("M,N,K,bs,dq,qt,seed", _cases())
def test_random_shape(M, N, K, bs, dq, qt, seed):
    note(f"random shape M={M} N={N} K={K} bs={bs} dq={dq} {qt}")
    dg = lib()
    d = dev()
    W = synth.normal((N, K), 0.02, seed, torch.bfloat16)
    X = synth.normal((M, K), 1.0, seed + 1)
    dY = synth.normal((M, N), 1.0, seed + 2)
    q = dg.nf4_quantize(W.to(d), blocksize=bs, double_quant=dq, quant_type=qt)
    Xd, dYd = X.to(d), dY.to(d)
    y32 = dg.nf4_matmul_fwd(Xd, q)
    y16 = dg.nf4_matmul_fwd(Xd, q, torch.bfloat16)
    dx32 = dg.nf4_matmul_bwd_dx(dYd, q)
    torch.cuda.synchronize()
    qo = O.quantize(W.float().numpy(), blocksize=bs, double_quant_on=dq, quant_type=qt)
    wh = O.bf16_bits_to_f32(O.dequantize(qo)).reshape(N, K).astype(np.float64)
    assert np.array_equal(bf16_bits(y16), O.f32_to_bf16_bits(y32.cpu().numpy()))
    x, dy = X.float().numpy(), dY.float().numpy()
    where = f"M={M} N={N} K={K} bs={bs} dq={dq} {qt}"
    assert_gemm_within_bound(y32, O.matmul_fwd(x, wh), O.fwd_bound(x, wh), f"fwd {where}")
    assert_gemm_within_bound(dx32, O.matmul_bwd_dx(dy, wh), O.bwd_dx_bound(dy, wh), f"bwd {where}")


def _lora_cases(n=16, seed=20261204):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        M = int(rng.choice([int(rng.integers(1, 17)), int(rng.integers(17, 260)), int(rng.integers(260, 700))]))
        N = int(rng.integers(1, 4001))
        if i % 2 == 0:
            N = max(8, N - N % 8)             # the transposing backward
        K = 64 * int(rng.integers(1, 13))
        r = 16 * int(rng.integers(1, 9))
        bs = int(rng.choice([32, 64, 128, 256]))
        dq = bool(rng.integers(0, 2))
        qt = "fp4" if rng.random() < 0.3 else "nf4"
        out.append((M, N, K, r, bs, dq, qt, 6000 + i))
    return out


@pytest.mark.parametrize("M,N,K,r,bs,dq,qt,seed", _lora_cases())
def test_random_shape_with_adapter(M, N, K, r, bs, dq, qt, seed):
    """"bitsandbytes" page, 4-bit/LoRA paragraph: the adapter term added in the same accumulators, on
    random shapes and formats (every kernel's adapter instantiation with the block sizes, codebooks
    and double-quantization settings drawn); bf16 outputs must be the one rounding of fp32."""
    note(f"random shape + adapter M={M} N={N} K={K} r={r} bs={bs} dq={dq} {qt}")
    dg = lib()
    d = dev()
    W = synth.normal((N, K), 0.02, seed, torch.bfloat16)
    X = synth.normal((M, K), 1.0, seed + 1)
    U = synth.normal((M, r), 1.0, seed + 2)
    B = synth.normal((N, r), 0.1, seed + 3)
    dY = synth.normal((M, N), 1.0, seed + 4)
    V = synth.normal((M, r), 1.0, seed + 5)
    At = synth.normal((K, r), 0.1, seed + 6)
    q = dg.nf4_quantize(W.to(d), blocksize=bs, double_quant=dq, quant_type=qt)
    y32 = dg.nf4_matmul_fwd_lora(X.to(d), q, U.to(d), B.to(d))
    y16 = dg.nf4_matmul_fwd_lora(X.to(d), q, U.to(d), B.to(d), torch.bfloat16)
    dx32 = dg.nf4_matmul_bwd_dx_lora(dY.to(d), q, V.to(d), At.to(d))
    dx16 = dg.nf4_matmul_bwd_dx_lora(dY.to(d), q, V.to(d), At.to(d), torch.bfloat16)
    torch.cuda.synchronize()
    qo = O.quantize(W.float().numpy(), blocksize=bs, double_quant_on=dq, quant_type=qt)
    wh = O.bf16_bits_to_f32(O.dequantize(qo)).reshape(N, K).astype(np.float64)
    assert np.array_equal(bf16_bits(y16), O.f32_to_bf16_bits(y32.cpu().numpy()))
    assert np.array_equal(bf16_bits(dx16), O.f32_to_bf16_bits(dx32.cpu().numpy()))
    x, u, b = X.float().numpy(), U.float().numpy(), B.float().numpy()
    dy, v, at = dY.float().numpy(), V.float().numpy(), At.float().numpy()
    where = f"M={M} N={N} K={K} r={r} bs={bs} dq={dq} {qt}"
    assert_gemm_within_bound(y32, O.matmul_fwd_lora(x, wh, u, b), O.fwd_lora_bound(x, wh, u, b), f"fwd+adapter {where}")
    assert_gemm_within_bound(dx32, O.matmul_bwd_dx_lora(dy, wh, v, at), O.bwd_dx_lora_bound(dy, wh, v, at),
                             f"bwd+adapter {where}")
