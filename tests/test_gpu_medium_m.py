"""GPU parity: the streaming forward over 16-row grid rows (M above 16).

"Zenbit" page, zenbit.pallas_nf4 bullet: the forward Y = X W^T with the
weight dequantized on chip.  From 17 rows up to (grid rows) x N = 14 * 4096
the forward keeps the small-M kernel and gives each 16 rows of X a grid row
of their own (the 256x256 kernel would leave most CUs idle there).  These
cases cover a last grid row of one row, X staged in LDS or read from memory
(K % 512), block size 32, bf16 output, the adapter term and the boundary of
the rule on both sides.  Every element is compared with the oracle's float64
product at 1e-4 * (|X| |W^|^T) (plus the adapter's term).
"""
import numpy as np
import pytest
import torch

import oracle as O
import synth
from tests._gpu import assert_gemm_within_bound, bf16_bits, dev, lib, note


pytestmark = pytest.mark.gpu


def _case(M, N, K, seed, bs=64, dq=True, qt="nf4"):
    dg = lib()
    W = synth.normal((N, K), 0.02, seed, torch.bfloat16)
    X = synth.normal((M, K), 1.0, seed + 1)
    q = dg.nf4_quantize(W.to(dev()), blocksize=bs, double_quant=dq, quant_type=qt)
    qo = O.quantize(W.float().numpy(), blocksize=bs, double_quant_on=dq, quant_type=qt)
    wh = O.bf16_bits_to_f32(O.dequantize(qo)).reshape(N, K).astype(np.float64)
    return dg, q, X, wh


@pytest.mark.parametrize("M,N,K", [
    (17, 4096, 4096),    # two grid rows, the second of one row; X staged in LDS
    (33, 1000, 1024),    # three grid rows, N not a multiple of 16
    (100, 2048, 320),    # seven grid rows, X read from memory (K % 512 != 0)
    (224, 4096, 512),    # 14 grid rows x 4096: the last shape of the rule
    (225, 4096, 512),    # 15 grid rows: the 256x256 kernel
    (256, 256, 2048),    # 16 grid rows of 16 columns
])
def test_grid_rows_every_element(M, N, K):
    note(f"medium M fwd {M}x{N}x{K}")
    dg, q, X, wh = _case(M, N, K, 5 * M + N + K)
    Y = dg.nf4_matmul_fwd(X.to(dev()), q)
    torch.cuda.synchronize()
    x = X.float().numpy()
    assert_gemm_within_bound(Y, O.matmul_fwd(x, wh), O.fwd_bound(x, wh), f"medium M {M}x{N}x{K}")


@pytest.mark.parametrize("bs,qt", [(32, "nf4"), (64, "fp4")])
def test_formats_and_bf16_output(bs, qt):
    M, N, K = 40, 1200, 1536
    note(f"medium M fwd bs={bs} {qt}")
    dg, q, X, wh = _case(M, N, K, 71 + bs, bs, True, qt)
    Xd = X.to(dev())
    y32 = dg.nf4_matmul_fwd(Xd, q)
    y16 = dg.nf4_matmul_fwd(Xd, q, torch.bfloat16)
    torch.cuda.synchronize()
    assert np.array_equal(bf16_bits(y16), O.f32_to_bf16_bits(y32.cpu().numpy()))
    x = X.float().numpy()
    assert_gemm_within_bound(y32, O.matmul_fwd(x, wh), O.fwd_bound(x, wh), f"medium M bs={bs} {qt}")


def test_adapter_term():
    M, N, K, r = 50, 800, 1024, 48
    note("medium M fwd + adapter")
    dg, q, X, wh = _case(M, N, K, 991)
    U = synth.normal((M, r), 1.0, 992)
    B = synth.normal((N, r), 0.1, 993)
    d = dev()
    Y = dg.nf4_matmul_fwd_lora(X.to(d), q, U.to(d), B.to(d))
    torch.cuda.synchronize()
    x, u, b = X.float().numpy(), U.float().numpy(), B.float().numpy()
    assert_gemm_within_bound(Y, O.matmul_fwd_lora(x, wh, u, b), O.fwd_lora_bound(x, wh, u, b), "medium M + adapter")
