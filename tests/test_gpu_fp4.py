"""GPU parity for the FP4 level table (quant_type="fp4").

"bitsandbytes" page, 4-bit training paragraph: the 4-bit data type is NF4 or
FP4, standard floating-point 4-bit.  FP4 codes are the E2M1 bit patterns and
their levels the values over 6; the quantizer, the dequantizer and every GEMM
run the same calls with that table.  Codes, packed bytes, absmax state and W^
bit-exact against the oracle run with the FP4 table (block sizes 32-256,
double quantization on and off, bf16 and fp32 weights); exact ties, threshold
neighbours, signed zeros and subnormals; the fused GEMMs within the stated
bound, and an identity input that must reproduce W^ exactly.
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
    qo = O.quantize(W_cpu.float().numpy(), blocksize=bs, double_quant_on=dq, quant_type="fp4")
    qg = dg.nf4_quantize(W_cpu.to(dev()), blocksize=bs, double_quant=dq, quant_type="fp4")
    torch.cuda.synchronize()
    assert qg.quant_type == "fp4"
    return dg, qg, qo


def _check_dequantize(dg, qg, qo, shape, where):
    wh = dg.nf4_dequantize(qg, torch.bfloat16)
    wf = dg.nf4_dequantize(qg, torch.float32)
    torch.cuda.synchronize()
    assert np.array_equal(bf16_bits(wh), O.dequantize(qo).reshape(shape)), where
    assert np.array_equal(u32(wf), O.dequantize(qo, out="f32").reshape(shape).view(np.uint32)), where


@pytest.mark.parametrize("bs", [32, 64, 128, 256])
@pytest.mark.parametrize("rows,cols", [(1, 1), (3, 37), (33, 65), (300, 777), (129, 4096)])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_quantize_dequantize_bit_exact(bs, rows, cols, dtype):
    W = synth.normal((rows, cols), 0.02, 400 + bs + rows + cols, dtype)
    for dq in (True, False):
        where = f"fp4 bs={bs} {rows}x{cols} {dtype} dq={dq}"
        dg, qg, qo = _quant(W, bs, dq)
        assert_quant_equal(qg, qo, where)
        _check_dequantize(dg, qg, qo, (rows, cols), where)


def _special_weight():
    """Blocks of 64 whose first element sets the absmax; the rest sit on every FP4 decision
    midpoint, its float32 neighbours, signed zeros and tiny values, at several scales."""
    c = O.fp4_codebook()
    vals = []
    for i in range(7):
        mid = (float(c[i]) + float(c[i + 1])) / 2        # exact in float64
        for v in (mid, -mid):
            f = np.float32(v)
            vals += [f, np.nextafter(f, np.float32(2)), np.nextafter(f, np.float32(-2))]
    vals += [0.0, -0.0, 1e-45, -1e-45, 1e-38, -1e-38, 0.125, -0.125, 1.0, -1.0, 0.5, -0.5]
    vals = np.array(vals, np.float32)
    rows = []
    for scale in (1.0, 2.0 ** -10, 3.7, 2.0 ** 100, 1e-30):
        body = (vals * np.float32(scale)).astype(np.float32)
        for start in range(0, body.size, 63):
            blk = np.zeros(64, np.float32)
            blk[0] = np.float32(scale)
            seg = body[start:start + 63]
            blk[1:1 + seg.size] = seg
            rows.append(blk)
    rows.append(np.zeros(64, np.float32))                       # all-zero block
    rows.append(np.full(64, -0.0, np.float32))                  # all -0
    last = np.zeros(64, np.float32)
    last[5], last[6] = -0.25, -0.0
    rows.append(last)
    return torch.from_numpy(np.concatenate(rows).reshape(-1, 64))


@pytest.mark.parametrize("dq", [True, False])
def test_ties_zeros_and_threshold_neighbours(dq):
    W = _special_weight()
    dg, qg, qo = _quant(W, 64, dq)
    assert_quant_equal(qg, qo, f"fp4 special dq={dq}")
    _check_dequantize(dg, qg, qo, tuple(W.shape), f"fp4 special dq={dq}")
    codes = O.unpack_codes(qg.packed.cpu().numpy(), W.numel()).reshape(W.shape)
    assert np.all(codes[-3] == 0) and np.all(codes[-2] == 0)    # zero blocks: code 0 (+0)
    assert codes[-1, 5] == 15 and codes[-1, 6] == 0             # -0.25 is the absmax: -1; a -0 beside it


def test_tail_block_and_odd_count():
    W = synth.normal((1, 64 * 5 + 29), 0.02, 431, torch.float32)    # partial last block, odd element count
    for bs in (32, 64, 256):
        dg, qg, qo = _quant(W, bs, True)
        assert_quant_equal(qg, qo, f"fp4 tail bs={bs}")
        _check_dequantize(dg, qg, qo, tuple(W.shape), f"fp4 tail bs={bs}")


@pytest.mark.parametrize("M,N,K", [
    (1, 256, 320), (16, 4096, 4096),                 # small-M forward
    (300, 264, 320), (513, 136, 1024),               # large-M forward, transposing backward
    (100, 300, 192),                                 # generic backward (N % 8 != 0)
])
def test_gemms_within_bound(M, N, K):
    note(f"fp4 M={M} N={N} K={K}")
    W = synth.normal((N, K), 0.02, 440 + M + N, torch.bfloat16)
    X = synth.normal((M, K), 1.0, 441 + M)
    dY = synth.normal((M, N), 1.0, 442 + M)
    dg, qg, qo = _quant(W, 64, True)
    d = dev()
    Y = dg.nf4_matmul_fwd(X.to(d), qg)
    dX = dg.nf4_matmul_bwd_dx(dY.to(d), qg)
    torch.cuda.synchronize()
    wh = O.bf16_bits_to_f32(O.dequantize(qo)).reshape(N, K)
    x, dy = X.float().numpy(), dY.float().numpy()
    assert_gemm_within_bound(Y, O.matmul_fwd(x, wh), O.fwd_bound(x, wh), f"fp4 fwd {M}x{N}x{K}")
    assert_gemm_within_bound(dX, O.matmul_bwd_dx(dy, wh), O.bwd_dx_bound(dy, wh), f"fp4 bwd {M}x{N}x{K}")


def test_identity_gemm_reproduces_dequantized_weight():
    """X = I: the fused forward must reproduce the FP4 W^ exactly (small and large M)."""
    N, K = 192, 256
    W = synth.normal((N, K), 0.02, 450, torch.bfloat16)
    dg, qg, qo = _quant(W, 64, True)
    d = dev()
    for M in (K, 16):
        X = torch.eye(K, dtype=torch.bfloat16)[:M].contiguous()
        Y = dg.nf4_matmul_fwd(X.to(d), qg)
        torch.cuda.synchronize()
        want = O.bf16_bits_to_f32(O.dequantize(qo)).reshape(N, K).T[:M]
        assert np.array_equal(Y.cpu().numpy(), want), M


def test_adapter_term_with_fp4_weight():
    M, N, K, r = 300, 256, 320, 32
    W = synth.normal((N, K), 0.02, 460, torch.bfloat16)
    X, U, B = synth.normal((M, K), 1.0, 461), synth.normal((M, r), 1.0, 462), synth.normal((N, r), 0.1, 463)
    dg, qg, qo = _quant(W, 64, True)
    d = dev()
    Y = dg.nf4_matmul_fwd_lora(X.to(d), qg, U.to(d), B.to(d))
    torch.cuda.synchronize()
    wh = O.bf16_bits_to_f32(O.dequantize(qo)).reshape(N, K)
    x, u, b = X.float().numpy(), U.float().numpy(), B.float().numpy()
    assert_gemm_within_bound(Y, O.matmul_fwd_lora(x, wh, u, b), O.fwd_lora_bound(x, wh, u, b), "fp4 lora fwd")


def test_nf4_and_fp4_share_the_absmax_state():
    W = synth.normal((64, 1024), 0.02, 470, torch.bfloat16)
    dg = lib()
    a = dg.nf4_quantize(W.to(dev()), quant_type="nf4")
    b = dg.nf4_quantize(W.to(dev()), quant_type="fp4")
    torch.cuda.synchronize()
    for f in ("absmax_q", "absmax_scale", "absmax_mean"):
        assert torch.equal(getattr(a, f), getattr(b, f)), f
    assert not torch.equal(a.packed, b.packed)


def test_linear_layer_and_device_save_load(tmp_path):
    from dequant_gemm_amd.io import load_qtensors, save_qtensors
    from dequant_gemm_amd.nn import NF4Linear
    dg, d = lib(), dev()
    N, K, M = 256, 320, 40
    W = synth.normal((N, K), 0.02, 480, torch.bfloat16)
    layer = NF4Linear.from_weight(W.to(d), out_dtype=torch.float32, quant_type="fp4")
    assert layer.qweight.quant_type == "fp4"
    X = synth.normal((M, K), 1.0, 481).to(d).requires_grad_(True)
    Y = layer(X)
    Y.backward(torch.ones_like(Y))
    torch.cuda.synchronize()
    qo = O.quantize(W.float().numpy(), 64, True, "fp4")
    wh = O.bf16_bits_to_f32(O.dequantize(qo)).reshape(N, K)
    x, g = X.detach().float().cpu().numpy(), np.ones((M, N), np.float32)
    assert_gemm_within_bound(Y, O.matmul_fwd(x, wh), O.fwd_bound(x, wh), "fp4 layer fwd")
    # the layer's gradient is bf16: allow its one rounding on top of the bound
    ref = O.matmul_bwd_dx(g, wh)
    assert_gemm_within_bound(X.grad, ref, O.bwd_dx_bound(g, wh) + np.abs(ref) * 2.0 ** -8, "fp4 layer dX (bf16)")
    p = str(tmp_path / "fp4.safetensors")
    save_qtensors(p, {"w": layer.qweight})
    back = load_qtensors(p, device=d)["w"]
    assert back.quant_type == "fp4"
    assert torch.equal(dg.nf4_dequantize(back), dg.nf4_dequantize(layer.qweight))
