"""GPU parity: the adapter's dense products (nf4_adapter_matmul) against the oracle.

"bitsandbytes" page, 4-bit/LoRA paragraph: a frozen 4-bit base weight with
small trainable low-rank adapters.  The adapter's down projection U = s X A^T,
the input gradient's activation V = s dY B and the adapter gradients
dA = V^T X and dB = dY^T U are compared element by element with the oracle's
float64 products at 1e-4 * |s| (|P| |Q|); the bf16 output must be one
round-to-nearest-even rounding of the fp32 output.
"""
import numpy as np
import pytest
import torch

import oracle as O
import synth
from tests._gpu import assert_gemm_within_bound, bf16_bits, dev, lib, note

pytestmark = pytest.mark.gpu


def _f64(t):
    return t.float().cpu().numpy().astype(np.float64)


def _four(M, N, K, r, s, seed):
    """The four adapter products on the GPU (fp32 outputs) and their oracle references."""
    dg = lib()
    d = dev()
    X = synth.normal((M, K), 1.0, seed)
    A = synth.normal((r, K), 0.05, seed + 1)
    dY = synth.normal((M, N), 1.0, seed + 2)
    B = synth.normal((N, r), 0.05, seed + 3)
    Xd, Ad, dYd, Bd = X.to(d), A.to(d), dY.to(d), B.to(d)
    U = dg.nf4_adapter_matmul(Xd, Ad, trans_b=True, alpha=s)
    V = dg.nf4_adapter_matmul(dYd, Bd, alpha=s)
    Ub, Vb = U.to(torch.bfloat16), V.to(torch.bfloat16)          # inputs of the gradients (layout only)
    dA = dg.nf4_adapter_matmul(Vb, Xd, trans_a=True)
    dB = dg.nf4_adapter_matmul(dYd, Ub, trans_a=True)
    torch.cuda.synchronize()
    x, a, dy, b = _f64(X), _f64(A), _f64(dY), _f64(B)
    u, v = _f64(Ub), _f64(Vb)
    return [
        (U, O.adapter_down(x, a, s), O.product_bound(x, a.T, s), "U = s X A^T"),
        (V, O.adapter_down_grad(dy, b, s), O.product_bound(dy, b, s), "V = s dY B"),
        (dA, O.adapter_grad_down(v, x), O.product_bound(v.T, x), "dA = V^T X"),
        (dB, O.adapter_grad_up(dy, u), O.product_bound(dy.T, u), "dB = dY^T U"),
    ]


@pytest.mark.parametrize("M,N,K,r", [
    (1, 64, 64, 16), (5, 300, 320, 48), (64, 64, 64, 64), (100, 513, 192, 16),
    (513, 136, 1024, 64), (1000, 88, 4096, 32), (17, 4096, 256, 128), (256, 256, 512, 1024),
])
def test_adapter_products_every_element(M, N, K, r):
    note(f"adapter products M={M} N={N} K={K} r={r}")
    for got, ref, bound, what in _four(M, N, K, r, 0.75, 7 * M + N + K + r):
        assert_gemm_within_bound(got, ref, bound, f"{what} M={M} N={N} K={K} r={r}")


def test_prefill_shape_rank64_every_element():
    """The adapter products of a rank-64 adapter on the prefill layer (M = K = 4096, N = 11008)."""
    note("adapter products at the prefill shape, rank 64")
    for got, ref, bound, what in _four(synth.PREFILL_M, synth.PREFILL_N, synth.PREFILL_K, 64, 2.0, 2100):
        assert_gemm_within_bound(got, ref, bound, f"prefill {what}")


@pytest.mark.parametrize("ta,tb", [(0, 0), (0, 1), (1, 0), (1, 1)])
def test_bf16_output_is_one_rounding_and_views_with_row_strides(ta, tb):
    dg = lib()
    d = dev()
    M, N, K = 96, 80, 200
    big_a = synth.normal((K + 8, M + 24) if ta else (M + 8, K + 24), 1.0, 31).to(d)
    big_b = synth.normal((N + 8, K + 24) if tb else (K + 8, N + 24), 1.0, 32).to(d)
    # row-strided views: rows padded by 24 elements
    A = big_a[:K, :M] if ta else big_a[:M, :K]
    B = big_b[:N, :K] if tb else big_b[:K, :N]
    c32 = dg.nf4_adapter_matmul(A, B, trans_a=bool(ta), trans_b=bool(tb), alpha=0.5)
    c16 = dg.nf4_adapter_matmul(A, B, trans_a=bool(ta), trans_b=bool(tb), alpha=0.5, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert np.array_equal(bf16_bits(c16), O.f32_to_bf16_bits(c32.cpu().numpy()))
    a, b = _f64(A), _f64(B)
    p, q = (a.T if ta else a), (b.T if tb else b)
    assert_gemm_within_bound(c32, 0.5 * (p @ q), O.product_bound(p, q, 0.5), f"views ta={ta} tb={tb}")


def test_empty_is_a_noop_and_bad_shapes_raise():
    dg = lib()
    d = dev()
    e = dg.nf4_adapter_matmul(torch.empty((0, 64), dtype=torch.bfloat16, device=d),
                              torch.empty((16, 64), dtype=torch.bfloat16, device=d), trans_b=True)
    assert e.shape == (0, 16)
    with pytest.raises(ValueError):
        dg.nf4_adapter_matmul(torch.empty((4, 64), dtype=torch.bfloat16, device=d),
                              torch.empty((32, 16), dtype=torch.bfloat16, device=d))
