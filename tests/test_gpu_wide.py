"""GPU parity: the one-wave-per-SIMD forward at its edges.

"Zenbit" page, zenbit.pallas_nf4 bullet: the forward Y = X W^T with the
weight dequantized on chip.  At block size 64 without an adapter term and K a
multiple of 256, the large-M forward runs a kernel with four waves of 64
output columns each, whose lanes each own a whole 64-block of a weight row per
128-K double step.  These cases cover its eight instantiations (fp32 or bf16
output, with and without double quantization, NF4 and FP4 codebooks), tiles cut
by M and N (waves with no rows, waves with no or a few columns), a single pair
of double steps, and K = 384 (odd double steps: the eight-wave kernel).  Every
element is compared with the oracle's float64 product at 1e-4 * (|X| |W^|^T);
bf16 outputs must be the one rounding of the fp32 result.
"""
import numpy as np
import pytest
import torch

import oracle as O
import synth
from tests._gpu import assert_gemm_within_bound, bf16_bits, dev, lib, note


pytestmark = pytest.mark.gpu


def _case(M, N, K, seed, dq, qt):
    dg = lib()
    W = synth.normal((N, K), 0.02, seed, torch.bfloat16)
    X = synth.normal((M, K), 1.0, seed + 1)
    q = dg.nf4_quantize(W.to(dev()), double_quant=dq, quant_type=qt)
    qo = O.quantize(W.float().numpy(), blocksize=64, double_quant_on=dq, quant_type=qt)
    wh = O.bf16_bits_to_f32(O.dequantize(qo)).reshape(N, K).astype(np.float64)
    return dg, q, X, wh


@pytest.mark.parametrize("qt", ["nf4", "fp4"])
@pytest.mark.parametrize("dq", [True, False])
def test_every_instantiation_on_a_cut_tile(dq, qt):
    # M = 300: the second row tile has 44 rows (one wave's worth, the other three
    # waves load zeros); N = 328: the second column tile has one full wave, one
    # wave of 8 columns and two waves past N; K = 768: three pairs of double steps
    M, N, K = 300, 328, 768
    note(f"wide fwd dq={dq} {qt} {M}x{N}x{K}")
    dg, q, X, wh = _case(M, N, K, 1000 + 10 * dq + (qt == "fp4"), dq, qt)
    Xd = X.to(dev())
    y32 = dg.nf4_matmul_fwd(Xd, q)
    y16 = dg.nf4_matmul_fwd(Xd, q, torch.bfloat16)
    torch.cuda.synchronize()
    assert np.array_equal(bf16_bits(y16), O.f32_to_bf16_bits(y32.cpu().numpy()))
    x = X.float().numpy()
    assert_gemm_within_bound(y32, O.matmul_fwd(x, wh), O.fwd_bound(x, wh), f"wide fwd dq={dq} {qt}")


@pytest.mark.parametrize("M,N,K", [
    (256, 256, 256),     # one whole tile, one pair of double steps
    (512, 768, 512),     # whole tiles in both directions
    (257, 65, 1024),     # one row and one column past a tile
    (17, 1000, 2304),    # a single partial row tile; nine pairs
    (600, 300, 384),     # K = 384: three double steps, the eight-wave kernel
])
def test_shapes(M, N, K):
    note(f"wide fwd {M}x{N}x{K}")
    dg, q, X, wh = _case(M, N, K, 7 * M + N + K, True, "nf4")
    Y = dg.nf4_matmul_fwd(X.to(dev()), q)
    torch.cuda.synchronize()
    x = X.float().numpy()
    assert_gemm_within_bound(Y, O.matmul_fwd(x, wh), O.fwd_bound(x, wh), f"wide fwd {M}x{N}x{K}")


def test_identity_rows_reproduce_the_weight():
    """X = rows of I: each output row is a dequantized weight column, exactly (K = 512)."""
    N, K = 320, 512
    dg, q, _, wh = _case(64, N, K, 4321, True, "nf4")
    X = torch.eye(K, dtype=torch.bfloat16)[100:400].contiguous()
    Y = dg.nf4_matmul_fwd(X.to(dev()), q)
    torch.cuda.synchronize()
    assert np.array_equal(Y.cpu().numpy(), wh.T[100:400].astype(np.float32))
