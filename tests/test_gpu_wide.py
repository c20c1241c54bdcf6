"""GPU parity: the one-wave-per-SIMD GEMM kernels at their edges.

"Zenbit" page, zenbit.pallas_nf4 bullet: the forward Y = X W^T and the
backward dX = dY W^ with the weight dequantized on chip.  When the 16-row
grid rows of the streaming kernel times N exceed 14 * 4096 the forward runs
four waves of 64 output columns whose lanes each own a whole
64-element chunk of a weight row per 128-K double step; the backward (N % 8
== 0) runs four waves of 64 output columns that dequantize 64-column weight
rows into a per-wave LDS tile.  "bitsandbytes" page, double-quantization
paragraph (block sizes) and 4-bit/LoRA paragraph (the adapter term).

These cases cover the forward's instantiations (fp32 or bf16 output, with and
without double quantization, NF4 and FP4 codebooks, block size 32 with two
blocks per chunk, the adapter term), tiles cut by M and N (waves with no rows,
waves with no or a few columns), K from one chunk (K = 64) to odd chunk and
double-step counts (zero-weight padding), and the backward's block-size-32
and adapter variants.  Every element is compared with the oracle's float64
product at 1e-4 * (|A| |B|) (plus the adapter's term); bf16 outputs must be
the one rounding of the fp32 result.
"""
import numpy as np
import pytest
import torch

import oracle as O
import synth
from tests._gpu import assert_gemm_within_bound, bf16_bits, dev, lib, note


pytestmark = pytest.mark.gpu


def _case(M, N, K, seed, dq=True, qt="nf4", bs=64):
    dg = lib()
    W = synth.normal((N, K), 0.02, seed, torch.bfloat16)
    X = synth.normal((M, K), 1.0, seed + 1)
    q = dg.nf4_quantize(W.to(dev()), blocksize=bs, double_quant=dq, quant_type=qt)
    qo = O.quantize(W.float().numpy(), blocksize=bs, double_quant_on=dq, quant_type=qt)
    wh = O.bf16_bits_to_f32(O.dequantize(qo)).reshape(N, K).astype(np.float64)
    return dg, q, X, wh


@pytest.mark.parametrize("bs", [64, 32])
@pytest.mark.parametrize("qt", ["nf4", "fp4"])
@pytest.mark.parametrize("dq", [True, False])
def test_every_instantiation_on_a_cut_tile(dq, qt, bs):
    # M = 300: the second row tile has 44 rows (one wave's worth, the other three
    # waves load zeros); N = 3400: the last column tile has one full wave, one
    # wave of 8 columns and two waves past N; K = 768: three pairs of double
    # steps.  The backward of the same weight (N % 8 == 0) on dY [300, 3400].
    M, N, K = 300, 3400, 768
    note(f"wide fwd/bwd dq={dq} {qt} bs={bs} {M}x{N}x{K}")
    dg, q, X, wh = _case(M, N, K, 1000 + 10 * dq + (qt == "fp4") + bs, dq, qt, bs)
    dY = synth.normal((M, N), 1.0, 1100 + bs)
    Xd, dYd = X.to(dev()), dY.to(dev())
    y32 = dg.nf4_matmul_fwd(Xd, q)
    y16 = dg.nf4_matmul_fwd(Xd, q, torch.bfloat16)
    dx32 = dg.nf4_matmul_bwd_dx(dYd, q)
    dx16 = dg.nf4_matmul_bwd_dx(dYd, q, torch.bfloat16)
    torch.cuda.synchronize()
    assert np.array_equal(bf16_bits(y16), O.f32_to_bf16_bits(y32.cpu().numpy()))
    assert np.array_equal(bf16_bits(dx16), O.f32_to_bf16_bits(dx32.cpu().numpy()))
    x, dy = X.float().numpy(), dY.float().numpy()
    where = f"dq={dq} {qt} bs={bs}"
    assert_gemm_within_bound(y32, O.matmul_fwd(x, wh), O.fwd_bound(x, wh), f"wide fwd {where}")
    assert_gemm_within_bound(dx32, O.matmul_bwd_dx(dy, wh), O.bwd_dx_bound(dy, wh), f"wide bwd {where}")


@pytest.mark.parametrize("M,N,K", [
    (256, 4096, 256),    # one whole row of tiles, one pair of double steps
    (512, 2048, 512),    # whole tiles in both directions
    (257, 3585, 1024),   # one row and one column past a tile
    (17, 28800, 256),    # a single partial row tile
    (300, 3100, 2304),   # nine pairs
    (600, 1600, 384),    # three double steps and a padding one
    (300, 3100, 64),     # K = 64: one chunk, lane group 1 and the second double step all padding
    (300, 3073, 320),    # five chunks: the third double step's second half is padding
    (300, 33000, 256),   # 2 x 129 tiles: more tiles than CUs (a second round of workgroups, cut tiles)
])
def test_shapes(M, N, K):
    note(f"wide fwd {M}x{N}x{K}")
    dg, q, X, wh = _case(M, N, K, 7 * M + N + K)
    Y = dg.nf4_matmul_fwd(X.to(dev()), q)
    torch.cuda.synchronize()
    x = X.float().numpy()
    assert_gemm_within_bound(Y, O.matmul_fwd(x, wh), O.fwd_bound(x, wh), f"wide fwd {M}x{N}x{K}")


@pytest.mark.parametrize("bs", [128, 256])
def test_large_block_sizes(bs):
    """Block sizes above 64: one block per 64-element chunk, blocks spanning rows (K = 320)."""
    M, N, K = 280, 3300, 320
    note(f"wide fwd/bwd bs={bs}")
    dg, q, X, wh = _case(M, N, K, 1300 + bs, True, "nf4", bs)
    dY = synth.normal((M, N), 1.0, 1301 + bs)
    Y = dg.nf4_matmul_fwd(X.to(dev()), q)
    dX = dg.nf4_matmul_bwd_dx(dY.to(dev()), q)
    torch.cuda.synchronize()
    x, dy = X.float().numpy(), dY.float().numpy()
    assert_gemm_within_bound(Y, O.matmul_fwd(x, wh), O.fwd_bound(x, wh), f"wide fwd bs={bs}")
    assert_gemm_within_bound(dX, O.matmul_bwd_dx(dy, wh), O.bwd_dx_bound(dy, wh), f"wide bwd bs={bs}")


@pytest.mark.parametrize("bs,r", [(64, 48), (32, 128)])
def test_adapter_term_on_cut_tiles(bs, r):
    """The adapter term added in the same accumulators: ragged tiles, ranks over one staged chunk."""
    M, N, K = 300, 3080, 320
    note(f"wide fwd/bwd + adapter bs={bs} r={r}")
    dg, q, X, wh = _case(M, N, K, 1500 + bs + r, True, "nf4", bs)
    U = synth.normal((M, r), 1.0, 1501 + r)
    B = synth.normal((N, r), 0.1, 1502 + r)
    dY = synth.normal((M, N), 1.0, 1503 + r)
    V = synth.normal((M, r), 1.0, 1504 + r)
    At = synth.normal((K, r), 0.1, 1505 + r)
    d = dev()
    Y = dg.nf4_matmul_fwd_lora(X.to(d), q, U.to(d), B.to(d))
    y16 = dg.nf4_matmul_fwd_lora(X.to(d), q, U.to(d), B.to(d), torch.bfloat16)
    dX = dg.nf4_matmul_bwd_dx_lora(dY.to(d), q, V.to(d), At.to(d))
    torch.cuda.synchronize()
    assert np.array_equal(bf16_bits(y16), O.f32_to_bf16_bits(Y.cpu().numpy()))
    x, u, b = X.float().numpy(), U.float().numpy(), B.float().numpy()
    dy, v, at = dY.float().numpy(), V.float().numpy(), At.float().numpy()
    assert_gemm_within_bound(Y, O.matmul_fwd_lora(x, wh, u, b), O.fwd_lora_bound(x, wh, u, b),
                             f"wide fwd + adapter bs={bs} r={r}")
    assert_gemm_within_bound(dX, O.matmul_bwd_dx_lora(dy, wh, v, at), O.bwd_dx_lora_bound(dy, wh, v, at),
                             f"wide bwd + adapter bs={bs} r={r}")


def test_identity_rows_reproduce_the_weight():
    """X = rows of I: each output row is a dequantized weight column, exactly (K = 512)."""
    N, K = 3100, 512
    dg, q, _, wh = _case(64, N, K, 4321)
    X = torch.eye(K, dtype=torch.bfloat16)[100:400].contiguous()
    Y = dg.nf4_matmul_fwd(X.to(dev()), q)
    torch.cuda.synchronize()
    assert np.array_equal(Y.cpu().numpy(), wh.T[100:400].astype(np.float32))
