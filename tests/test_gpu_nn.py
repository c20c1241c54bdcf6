"""GPU: NF4Linear (autograd over the fused GEMMs) and the device save/load round trip.

"Zenbit" page, section "What's inside": the fused NF4 dense layer, whose custom
backward forms dL/dX only.  Checks: the layer's forward and backward are the
fused kernels' outputs bit for bit; the bf16 output of either kernel is the
round-to-nearest-even of its fp32 output (one rounding of the same
accumulator); the fp32 path meets the oracle's bound through autograd; a
weight saved and loaded back computes the same products.
"""
import numpy as np
import pytest
import torch

import oracle as O
import synth
from tests._gpu import assert_gemm_within_bound, bf16_bits, dev, lib, oracle_quantize

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("M,N,K", [(1, 256, 256), (7, 300, 320), (16, 512, 4096), (300, 700, 512), (1024, 1024, 1024)])
def test_bf16_output_is_one_rounding_of_fp32(M, N, K):
    dg = lib()
    d = dev()
    W = synth.normal((N, K), 0.02, 50 + M, torch.bfloat16).to(d)
    X = synth.normal((M, K), 1.0, 51 + M).to(d)
    dY = synth.normal((M, N), 1.0, 52 + M).to(d)
    q = dg.nf4_quantize(W)
    y32 = dg.nf4_matmul_fwd(X, q, torch.float32)
    y16 = dg.nf4_matmul_fwd(X, q, torch.bfloat16)
    d32 = dg.nf4_matmul_bwd_dx(dY, q, torch.float32)
    d16 = dg.nf4_matmul_bwd_dx(dY, q, torch.bfloat16)
    torch.cuda.synchronize()
    assert np.array_equal(bf16_bits(y16), bf16_bits(y32.to(torch.bfloat16))), "fwd bf16 epilogue"
    assert np.array_equal(bf16_bits(d16), bf16_bits(d32.to(torch.bfloat16))), "bwd bf16 epilogue"


@pytest.mark.parametrize("lead", [(5,), (2, 3), (4, 64)])
def test_nf4linear_matches_fused_kernels(lead):
    dg = lib()
    from dequant_gemm_amd.nn import NF4Linear
    d = dev()
    N, K = 384, 512
    W = synth.normal((N, K), 0.02, 60, torch.bfloat16).to(d)
    layer = NF4Linear.from_weight(W)
    x = synth.normal((int(np.prod(lead)), K), 1.0, 61).to(d).reshape(*lead, K).requires_grad_(True)
    y = layer(x)
    assert y.shape == (*lead, N) and y.dtype == torch.bfloat16
    g = synth.normal((int(np.prod(lead)), N), 1.0, 62).to(d).reshape(*lead, N)
    y.backward(g)
    want_y = dg.nf4_matmul_fwd(x.detach().reshape(-1, K), layer.qweight, torch.bfloat16)
    want_dx = dg.nf4_matmul_bwd_dx(g.reshape(-1, N), layer.qweight, torch.bfloat16)
    torch.cuda.synchronize()
    assert np.array_equal(bf16_bits(y.reshape(-1, N)), bf16_bits(want_y)), "forward"
    assert x.grad.dtype == torch.bfloat16
    assert np.array_equal(bf16_bits(x.grad.reshape(-1, K)), bf16_bits(want_dx)), "backward"


def test_nf4linear_fp32_against_oracle():
    lib()
    from dequant_gemm_amd.nn import NF4Linear
    d = dev()
    N, K, M = 256, 320, 40
    W = synth.normal((N, K), 0.02, 70, torch.bfloat16)
    layer = NF4Linear.from_weight(W.to(d), out_dtype=torch.float32)
    X = synth.normal((M, K), 1.0, 71)
    x = X.to(d).reshape(4, 10, K).requires_grad_(True)
    y = layer(x)
    dY = synth.normal((M, N), 1.0, 72)
    y.backward(dY.to(d).float().reshape(4, 10, N))      # fp32 gradient: rounded to bf16 first (exact here)
    torch.cuda.synchronize()
    wh = O.bf16_bits_to_f32(O.dequantize(oracle_quantize(W, True))).reshape(N, K)
    xf, dyf = X.float().numpy(), dY.float().numpy()
    assert_gemm_within_bound(y.detach().reshape(M, N), O.matmul_fwd(xf, wh), O.fwd_bound(xf, wh), "fwd")
    # the layer's gradient is bf16: allow its one rounding on top of the bound
    ref = O.matmul_bwd_dx(dyf, wh)
    bound = O.bwd_dx_bound(dyf, wh) + np.abs(ref) * 2.0 ** -8
    assert_gemm_within_bound(x.grad.reshape(M, K), ref, bound, "bwd (bf16)")


def test_quantize_linears_and_no_weight_grad():
    lib()
    from dequant_gemm_amd.nn import NF4Linear, quantize_linears
    d = dev()
    torch.manual_seed(0)
    net = torch.nn.Sequential(torch.nn.Linear(128, 256, bias=False), torch.nn.GELU(),
                              torch.nn.Linear(256, 64, bias=False), torch.nn.Linear(64, 8))
    net = net.to(d).to(torch.bfloat16)
    quantize_linears(net)
    assert isinstance(net[0], NF4Linear) and isinstance(net[2], NF4Linear)
    assert isinstance(net[3], torch.nn.Linear)           # has a bias: left dense
    assert not any(p.requires_grad for p in net[0].parameters())
    x = torch.randn(3, 128, device=d, dtype=torch.bfloat16, requires_grad=True)
    net(x).float().sum().backward()
    torch.cuda.synchronize()
    assert x.grad is not None and torch.isfinite(x.grad.float()).all()


def test_device_save_load_round_trip(tmp_path):
    dg = lib()
    from dequant_gemm_amd.io import load_qtensors, save_qtensors
    d = dev()
    ws = {"a": dg.nf4_quantize(synth.normal((512, 256), 0.02, 80, torch.bfloat16).to(d)),
          "b": dg.nf4_quantize(synth.normal((33, 65), 0.02, 81, torch.float32).to(d), double_quant=False)}
    p = str(tmp_path / "q.safetensors")
    save_qtensors(p, ws)
    back = load_qtensors(p, device=d)
    X = synth.normal((20, 256), 1.0, 82).to(d)
    for k in ws:
        w0 = dg.nf4_dequantize(ws[k])
        w1 = dg.nf4_dequantize(back[k])
        torch.cuda.synchronize()
        assert np.array_equal(bf16_bits(w0), bf16_bits(w1)), k
    y0 = dg.nf4_matmul_fwd(X, ws["a"])
    y1 = dg.nf4_matmul_fwd(X, back["a"])
    torch.cuda.synchronize()
    assert torch.equal(y0, y1)


def test_nf4loralinear_forward_and_gradients():
    """The adapter layer against a float64 host evaluation of the same formula.

    y = x W^T + s (x A^T) B^T; dx = dy W^ + s (dy B) A; dA = s (dy B)^T x;
    dB = s dy^T (x A^T).  The kernels' parts are held to the 1e-4 bound; the
    layer's one bf16 rounding of y / dx and of the adapter activations U, V
    (each at most 2^-8 relative) is allowed on top.
    """
    lib()
    from dequant_gemm_amd.nn import NF4LoraLinear
    d = dev()
    N, K, M, r, alpha = 192, 256, 48, 16, 32.0
    W = synth.normal((N, K), 0.02, 90, torch.bfloat16)
    layer = NF4LoraLinear.from_weight(W.to(d), r, alpha)
    with torch.no_grad():
        layer.lora_b.copy_(synth.normal((N, r), 0.05, 91).to(d))
    X = synth.normal((M, K), 1.0, 92)
    x = X.to(d).reshape(6, 8, K).requires_grad_(True)
    y = layer(x)
    dY = synth.normal((M, N), 1.0, 93)
    y.backward(dY.to(d).reshape(6, 8, N))
    torch.cuda.synchronize()
    s = alpha / r
    wh = O.bf16_bits_to_f32(O.dequantize(oracle_quantize(W, True))).reshape(N, K).astype(np.float64)
    a = layer.lora_a.detach().float().cpu().numpy().astype(np.float64)
    b = layer.lora_b.detach().float().cpu().numpy().astype(np.float64)
    x64, dy64 = X.float().numpy().astype(np.float64), dY.float().numpy().astype(np.float64)
    xa, dyb = x64 @ a.T, dy64 @ b
    y_ref = x64 @ wh.T + s * xa @ b.T
    y_tol = 1e-4 * (np.abs(x64) @ np.abs(wh).T) + 2.0 ** -8 * (np.abs(y_ref) + s * np.abs(xa) @ np.abs(b).T)
    assert_gemm_within_bound(y.detach().reshape(M, N), y_ref, y_tol, "lora layer y")
    dx_ref = dy64 @ wh + s * dyb @ a
    dx_tol = 1e-4 * (np.abs(dy64) @ np.abs(wh)) + 2.0 ** -8 * (np.abs(dx_ref) + s * np.abs(dyb) @ np.abs(a))
    assert_gemm_within_bound(x.grad.reshape(M, K), dx_ref, dx_tol, "lora layer dx")
    da_ref, db_ref = s * dyb.T @ x64, s * dy64.T @ xa
    da_tol = 2.0 ** -7 * s * (np.abs(dyb).T @ np.abs(x64))
    db_tol = 2.0 ** -7 * s * (np.abs(dy64).T @ np.abs(xa))
    assert_gemm_within_bound(layer.lora_a.grad, da_ref, da_tol, "lora dA")
    assert_gemm_within_bound(layer.lora_b.grad, db_ref, db_tol, "lora dB")
