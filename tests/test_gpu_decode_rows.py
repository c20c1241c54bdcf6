"""GPU parity: the small-M forward over weights of many 16-row groups.

"Zenbit" page, zenbit.pallas_nf4 bullet: the forward Y = X W^T with the
weight dequantized on chip.  At M <= 16 and at least 1536 groups of 16 weight
rows (K <= 8192), the forward runs a kernel that keeps X in registers across
a run of row groups per workgroup.  These cases put it through its edges:
row-group counts that do not divide by the grid (one extra group on some
workgroups), N not a multiple of 16, K from one quantization block to 8192
(one or two blocks per lane and row, lanes with no block), every M from 1 to
16, block size 32, fp32 absmax, the FP4 codebook, bf16 output and the
adapter term.  Every output element is compared with the oracle's float64
product at 1e-4 * (|X| |W^|^T) (plus the adapter's term).
"""
import numpy as np
import pytest
import torch

import oracle as O
import synth
from tests._gpu import assert_gemm_within_bound, bf16_bits, dev, lib, note

pytestmark = pytest.mark.gpu


def _quantized(N, K, seed, bs=64, dq=True, qt="nf4"):
    dg = lib()
    W = synth.normal((N, K), 0.02, seed, torch.bfloat16)
    q = dg.nf4_quantize(W.to(dev()), blocksize=bs, double_quant=dq, quant_type=qt)
    qo = O.quantize(W.float().numpy(), blocksize=bs, double_quant_on=dq, quant_type=qt)
    wh = O.bf16_bits_to_f32(O.dequantize(qo)).reshape(N, K).astype(np.float64)
    return q, wh


@pytest.mark.parametrize("M,N,K", [
    (1, 24576, 64),        # 1536 groups: six per workgroup, one block per row (63 of 64 slots idle)
    (16, 24592, 1024),     # 1537 groups: one workgroup takes seven
    (7, 24583, 4096),      # N % 16 = 7: the last group is partial; one block per lane and row
    (3, 25000, 4160),      # two blocks per lane and row, the second only on slot 0
    (16, 26000, 8192),     # two blocks per lane and row, all slots busy
])
def test_rows_kernel_every_element(M, N, K):
    note(f"decode rows kernel M={M} N={N} K={K}")
    dg = lib()
    q, wh = _quantized(N, K, 11 * M + N + K)
    X = synth.normal((M, K), 1.0, 3 * M + K)
    Y = dg.nf4_matmul_fwd(X.to(dev()), q)
    torch.cuda.synchronize()
    x = X.float().numpy()
    assert_gemm_within_bound(Y, O.matmul_fwd(x, wh), O.fwd_bound(x, wh), f"rows M={M} N={N} K={K}")


@pytest.mark.parametrize("bs,dq,qt", [(32, True, "nf4"), (64, False, "nf4"), (32, False, "fp4"), (64, True, "fp4")])
def test_rows_kernel_formats(bs, dq, qt):
    N, K = 24600, 2048
    note(f"decode rows kernel bs={bs} dq={dq} {qt}")
    dg = lib()
    q, wh = _quantized(N, K, 77 + bs, bs, dq, qt)
    for M in (2, 16):
        X = synth.normal((M, K), 1.0, 80 + M)
        Y = dg.nf4_matmul_fwd(X.to(dev()), q)
        torch.cuda.synchronize()
        x = X.float().numpy()
        assert_gemm_within_bound(Y, O.matmul_fwd(x, wh), O.fwd_bound(x, wh), f"rows bs={bs} dq={dq} {qt} M={M}")


def test_rows_kernel_every_m():
    """M = 1 .. 16 on one weight: each count of X rows (the rest of the MFMA's rows are zeros)."""
    N, K = 24640, 512
    dg = lib()
    q, wh = _quantized(N, K, 501)
    for M in range(1, 17):
        note(f"decode rows kernel M={M}")
        X = synth.normal((M, K), 1.0, 600 + M)
        Y = dg.nf4_matmul_fwd(X.to(dev()), q)
        torch.cuda.synchronize()
        x = X.float().numpy()
        assert_gemm_within_bound(Y, O.matmul_fwd(x, wh), O.fwd_bound(x, wh), f"rows M={M}")


def test_rows_kernel_bf16_output_and_adapter():
    M, N, K, r = 5, 24592, 1536, 48
    note("decode rows kernel: bf16 output, adapter term")
    dg = lib()
    d = dev()
    q, wh = _quantized(N, K, 901)
    X = synth.normal((M, K), 1.0, 902)
    U = synth.normal((M, r), 1.0, 903)
    B = synth.normal((N, r), 0.1, 904)
    Xd, Ud, Bd = X.to(d), U.to(d), B.to(d)
    y32 = dg.nf4_matmul_fwd(Xd, q)
    y16 = dg.nf4_matmul_fwd(Xd, q, torch.bfloat16)
    l32 = dg.nf4_matmul_fwd_lora(Xd, q, Ud, Bd)
    l16 = dg.nf4_matmul_fwd_lora(Xd, q, Ud, Bd, torch.bfloat16)
    torch.cuda.synchronize()
    assert np.array_equal(bf16_bits(y16), O.f32_to_bf16_bits(y32.cpu().numpy()))
    assert np.array_equal(bf16_bits(l16), O.f32_to_bf16_bits(l32.cpu().numpy()))
    x, u, b = X.float().numpy(), U.float().numpy(), B.float().numpy()
    assert_gemm_within_bound(y32, O.matmul_fwd(x, wh), O.fwd_bound(x, wh), "rows fp32")
    assert_gemm_within_bound(l32, O.matmul_fwd_lora(x, wh, u, b), O.fwd_lora_bound(x, wh, u, b), "rows + adapter")
