"""GPU parity: the fused GEMMs with a low-rank adapter term, against the oracle.

"bitsandbytes" page, 4-bit/LoRA paragraph (frozen 4-bit base weight plus a
trainable low-rank adapter).  Y = X W^T + U B^T and dX = dY W^ + V A are
formed in one pass, the adapter product in the same fp32 accumulators; every
element must satisfy |err| <= 1e-4 * (|X||W^|^T + |U||B|^T) (resp. the
backward's terms).  Shapes cover the small-M forward (M <= 16), the large-M
forward, the transposing backward (N % 8 == 0) and the generic backward
(N % 8 != 0), ragged tiles and ranks 16 .. 128.
"""
import numpy as np
import pytest
import torch

import oracle as O
import synth
from tests._gpu import assert_gemm_within_bound, bf16_bits, dev, lib, note, oracle_quantize

pytestmark = pytest.mark.gpu


def _case(M, N, K, r, seed):
    dg = lib()
    d = dev()
    W = synth.normal((N, K), 0.02, seed, torch.bfloat16)
    X = synth.normal((M, K), 1.0, seed + 1)
    U = synth.normal((M, r), 1.0, seed + 2)
    B = synth.normal((N, r), 0.1, seed + 3)
    dY = synth.normal((M, N), 1.0, seed + 4)
    V = synth.normal((M, r), 1.0, seed + 5)
    At = synth.normal((K, r), 0.1, seed + 6)
    q = dg.nf4_quantize(W.to(d))
    return dg, d, W, X, U, B, dY, V, At, q


@pytest.mark.parametrize("M,N,K,r", [
    (1, 256, 256, 16), (5, 300, 320, 48), (16, 512, 4096, 64), (3, 17, 64, 32),      # small-M forward
    (17, 300, 256, 16), (256, 256, 512, 32), (300, 704, 512, 128), (513, 136, 1024, 64),  # large-M
    (1000, 88, 192, 16),
])
def test_lora_fwd_bwd_against_oracle(M, N, K, r):
    note(f"lora M={M} N={N} K={K} r={r}")
    dg, d, W, X, U, B, dY, V, At, q = _case(M, N, K, r, 9 * M + N + K + r)
    Y = dg.nf4_matmul_fwd_lora(X.to(d), q, U.to(d), B.to(d))
    dX = dg.nf4_matmul_bwd_dx_lora(dY.to(d), q, V.to(d), At.to(d))
    torch.cuda.synchronize()
    wh = O.bf16_bits_to_f32(O.dequantize(oracle_quantize(W, True))).reshape(N, K)
    x, u, b = X.float().numpy(), U.float().numpy(), B.float().numpy()
    dy, v, at = dY.float().numpy(), V.float().numpy(), At.float().numpy()
    assert_gemm_within_bound(Y, O.matmul_fwd_lora(x, wh, u, b), O.fwd_lora_bound(x, wh, u, b),
                             f"fwd+lora {M}x{N}x{K} r={r}")
    assert_gemm_within_bound(dX, O.matmul_bwd_dx_lora(dy, wh, v, at), O.bwd_dx_lora_bound(dy, wh, v, at),
                             f"bwd+lora {M}x{N}x{K} r={r}")


@pytest.mark.parametrize("M,N,K", [(4, 256, 512), (300, 512, 256), (64, 100, 128)])
def test_lora_bf16_output_and_zero_adapter(M, N, K):
    dg, d, W, X, U, B, dY, V, At, q = _case(M, N, K, 32, 500 + M)
    Xd, Ud, Bd, dYd, Vd, Atd = (t.to(d) for t in (X, U, B, dY, V, At))
    y32 = dg.nf4_matmul_fwd_lora(Xd, q, Ud, Bd)
    y16 = dg.nf4_matmul_fwd_lora(Xd, q, Ud, Bd, torch.bfloat16)
    d32 = dg.nf4_matmul_bwd_dx_lora(dYd, q, Vd, Atd)
    d16 = dg.nf4_matmul_bwd_dx_lora(dYd, q, Vd, Atd, torch.bfloat16)
    # a zero adapter leaves exactly the plain fused products
    y0 = dg.nf4_matmul_fwd_lora(Xd, q, torch.zeros_like(Ud), Bd)
    d0 = dg.nf4_matmul_bwd_dx_lora(dYd, q, torch.zeros_like(Vd), Atd)
    yp = dg.nf4_matmul_fwd(Xd, q)
    dp = dg.nf4_matmul_bwd_dx(dYd, q)
    torch.cuda.synchronize()
    assert np.array_equal(bf16_bits(y16), bf16_bits(y32.to(torch.bfloat16)))
    assert np.array_equal(bf16_bits(d16), bf16_bits(d32.to(torch.bfloat16)))
    assert torch.equal(y0, yp) and torch.equal(d0, dp)


def test_lora_prefill_shape_sampled_rows():
    """The prefill GEMM shape with a rank-64 adapter, on sampled rows."""
    dg = lib()
    d = dev()
    M, N, K, r = synth.PREFILL_M, synth.PREFILL_N, synth.PREFILL_K, 64
    W = synth.prefill_weight()
    X = synth.prefill_x()
    U = synth.normal((M, r), 1.0, 2100)
    B = synth.normal((N, r), 0.1, 2101)
    q = dg.nf4_quantize(W.to(d))
    Y = dg.nf4_matmul_fwd_lora(X.to(d), q, U.to(d), B.to(d))
    torch.cuda.synchronize()
    rows = np.array([0, 1, 255, 256, 2047, 4000, 4095])
    wh = O.bf16_bits_to_f32(O.dequantize(oracle_quantize(W, True))).reshape(N, K)
    x, u, b = X[rows].float().numpy(), U[rows].float().numpy(), B.float().numpy()
    assert_gemm_within_bound(Y[rows], O.matmul_fwd_lora(x, wh, u, b), O.fwd_lora_bound(x, wh, u, b), "prefill+lora")
