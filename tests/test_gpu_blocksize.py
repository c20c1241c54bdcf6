"""GPU parity for block sizes 32, 128 and 256 (64 is covered everywhere else).

The absmax block is 64 weights on the pages ("bitsandbytes" page, double
quantization paragraph); the same quantizer with 32, 128 or 256 weights per
block: codes, packed bytes, absmax state and W^ bit-exact against the oracle
run with that block size, and the fused GEMMs within the stated bound.  Shapes
include columns that are not a multiple of the block size, so blocks span
weight rows, odd element counts and partial last blocks.
"""
import numpy as np
import pytest
import torch

import oracle as O
import synth
from tests._gpu import assert_gemm_within_bound, assert_quant_equal, bf16_bits, dev, lib, note, u32

pytestmark = pytest.mark.gpu


def _quant(W_cpu, bs, dq):
    dg = lib()
    qo = O.quantize(W_cpu.float().numpy(), blocksize=bs, double_quant_on=dq)
    qg = dg.nf4_quantize(W_cpu.to(dev()), blocksize=bs, double_quant=dq)
    torch.cuda.synchronize()
    return dg, qg, qo


@pytest.mark.parametrize("bs", [32, 128, 256])
@pytest.mark.parametrize("rows,cols", [(1, 1), (3, 37), (7, 1000), (33, 65), (300, 777), (64, 320), (129, 4096)])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_quantize_dequantize_bit_exact(bs, rows, cols, dtype):
    W = synth.normal((rows, cols), 0.02, 300 + bs + rows + cols, dtype)
    for dq in (True, False):
        where = f"bs={bs} {rows}x{cols} {dtype} dq={dq}"
        dg, qg, qo = _quant(W, bs, dq)
        assert qg.blocksize == bs
        assert_quant_equal(qg, qo, where)
        wh = dg.nf4_dequantize(qg, torch.bfloat16)
        wf = dg.nf4_dequantize(qg, torch.float32)
        torch.cuda.synchronize()
        assert np.array_equal(bf16_bits(wh), O.dequantize(qo).reshape(rows, cols)), where
        assert np.array_equal(u32(wf), O.dequantize(qo, out="f32").reshape(rows, cols).view(np.uint32)), where


@pytest.mark.parametrize("bs", [32, 128, 256])
def test_heavy_tailed_large_weight(bs):
    W = synth.student_t((2048, 2048), 4.0, 0.02, 310 + bs)
    dg, qg, qo = _quant(W, bs, True)
    assert_quant_equal(qg, qo, f"student-t bs={bs}")
    wh = dg.nf4_dequantize(qg)
    torch.cuda.synchronize()
    assert np.array_equal(bf16_bits(wh), O.dequantize(qo).reshape(2048, 2048))


@pytest.mark.parametrize("bs", [32, 128, 256])
@pytest.mark.parametrize("M,N,K", [
    (1, 256, 320), (7, 300, 192), (16, 512, 4096),            # small-M forward (two tables per chunk at 32)
    (300, 264, 320), (513, 136, 1024), (256, 256, 4096),        # large-M forward, transposing backward
    (100, 300, 192),                                             # generic backward (N % 8 != 0)
])
def test_gemms_within_bound(bs, M, N, K):
    note(f"bs={bs} M={M} N={N} K={K}")
    W = synth.normal((N, K), 0.02, 320 + bs + M + N, torch.bfloat16)
    X = synth.normal((M, K), 1.0, 321 + M)
    dY = synth.normal((M, N), 1.0, 322 + M)
    dg, qg, qo = _quant(W, bs, True)
    d = dev()
    Y = dg.nf4_matmul_fwd(X.to(d), qg)
    dX = dg.nf4_matmul_bwd_dx(dY.to(d), qg)
    torch.cuda.synchronize()
    wh = O.bf16_bits_to_f32(O.dequantize(qo)).reshape(N, K)
    x, dy = X.float().numpy(), dY.float().numpy()
    assert_gemm_within_bound(Y, O.matmul_fwd(x, wh), O.fwd_bound(x, wh), f"fwd bs={bs} {M}x{N}x{K}")
    assert_gemm_within_bound(dX, O.matmul_bwd_dx(dy, wh), O.bwd_dx_bound(dy, wh), f"bwd bs={bs} {M}x{N}x{K}")


@pytest.mark.parametrize("bs", [32, 256])
def test_identity_gemm_reproduces_dequantized_weight(bs):
    """X = I: the fused forward must reproduce W^ (as dequantized) exactly."""
    N, K = 192, 256
    W = synth.normal((N, K), 0.02, 330 + bs, torch.bfloat16)
    dg, qg, qo = _quant(W, bs, True)
    d = dev()
    for M in (K, 16):
        X = torch.eye(K, dtype=torch.bfloat16)[:M].contiguous()
        Y = dg.nf4_matmul_fwd(X.to(d), qg)
        torch.cuda.synchronize()
        want = O.bf16_bits_to_f32(O.dequantize(qo)).reshape(N, K).T[:M]
        assert np.array_equal(Y.cpu().numpy(), want), (bs, M)


def test_adapter_term_with_other_block_size():
    M, N, K, r, bs = 300, 256, 320, 32, 32
    W = synth.normal((N, K), 0.02, 340, torch.bfloat16)
    X, U, B = synth.normal((M, K), 1.0, 341), synth.normal((M, r), 1.0, 342), synth.normal((N, r), 0.1, 343)
    dg, qg, qo = _quant(W, bs, True)
    d = dev()
    Y = dg.nf4_matmul_fwd_lora(X.to(d), qg, U.to(d), B.to(d))
    torch.cuda.synchronize()
    wh = O.bf16_bits_to_f32(O.dequantize(qo)).reshape(N, K)
    x, u, b = X.float().numpy(), U.float().numpy(), B.float().numpy()
    assert_gemm_within_bound(Y, O.matmul_fwd_lora(x, wh, u, b), O.fwd_lora_bound(x, wh, u, b), "lora bs=32")
