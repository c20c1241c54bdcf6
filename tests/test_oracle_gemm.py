"""Pins for the oracle's GEMM references and their per-element bound.

Method passages: "Zenbit" page, *What's inside*, ``zenbit.pallas_nf4`` bullet
(fused dequant+matmul forward; fused backward forming dL/dX only);
"bitsandbytes" page, quantized-GEMM paragraph (float32 multiply and output).
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle as O


def _bf16(rng, shape, std=1.0):
    return O.bf16_bits_to_f32(O.f32_to_bf16_bits((rng.standard_normal(shape) * std).astype(np.float32)))


def test_fwd_and_bwd_against_exact_rationals():
    rng = np.random.default_rng(0)
    M, N, K = 3, 5, 64
    x = _bf16(rng, (M, K))
    w = _bf16(rng, (N, K), 0.02)
    dy = _bf16(rng, (M, N))
    y = O.matmul_fwd(x, w)
    dx = O.matmul_bwd_dx(dy, w)
    for i in range(M):
        for j in range(N):
            exact = sum(Fraction(float(x[i, k])) * Fraction(float(w[j, k])) for k in range(K))
            assert abs(Fraction(float(y[i, j])) - exact) <= Fraction(K) * Fraction(2) ** -52 * \
                sum(abs(Fraction(float(x[i, k])) * Fraction(float(w[j, k]))) for k in range(K))
    for i in range(M):
        for k in range(K):
            exact = sum(Fraction(float(dy[i, j])) * Fraction(float(w[j, k])) for j in range(N))
            mag = sum(abs(Fraction(float(dy[i, j])) * Fraction(float(w[j, k]))) for j in range(N))
            assert abs(Fraction(float(dx[i, k])) - exact) <= Fraction(N) * Fraction(2) ** -52 * mag


def test_identity_special_cases_are_exact():
    rng = np.random.default_rng(1)
    q = O.quantize((rng.standard_normal(256 * 256) * 0.02).astype(np.float32))
    wh = O.bf16_bits_to_f32(O.dequantize(q)).reshape(256, 256)
    assert np.array_equal(O.matmul_fwd(np.eye(256, dtype=np.float32), wh), wh.T.astype(np.float64))
    assert np.array_equal(O.matmul_bwd_dx(np.eye(256, dtype=np.float32), wh), wh.astype(np.float64))


def test_bound_accepts_fp32_accumulation_and_rejects_mistakes():
    rng = np.random.default_rng(2)
    M, N, K = 16, 96, 4096
    x = _bf16(rng, (M, K))
    w = _bf16(rng, (N, K), 0.02)
    ref = O.matmul_fwd(x, w)
    bound = O.fwd_bound(x, w)
    # an fp32 accumulation in a different order passes
    acc = np.zeros((M, N), np.float32)
    for k0 in range(0, K, 64):
        acc += (x[:, k0:k0 + 64] @ w[:, k0:k0 + 64].T).astype(np.float32)
    assert O.gemm_violations(acc, ref, bound) == 0
    # a dropped K slice, a sign error, a transposed-operand mistake all fail
    acc_drop = acc - (x[:, :64] @ w[:, :64].T).astype(np.float32)
    assert O.gemm_violations(acc_drop, ref, bound) > 0
    assert O.gemm_violations(-acc, ref, bound) > 0
    wt = w.reshape(N, 64, K // 64).transpose(0, 2, 1).reshape(N, K)
    assert O.gemm_violations(O.matmul_fwd(x, wt), ref, bound) > 0


def test_bf16_rounded_outputs_would_break_the_bound():
    """Why the GEMM outputs are fp32: bf16 rounding of Y exceeds 1e-4 * |X||W|."""
    rng = np.random.default_rng(3)
    M, N, K = 8, 256, 4096
    x = _bf16(rng, (M, K))
    w = _bf16(rng, (N, K), 0.02)
    ref = O.matmul_fwd(x, w)
    y_bf16 = O.bf16_bits_to_f32(O.f32_to_bf16_bits(ref.astype(np.float32)))
    assert O.gemm_violations(y_bf16, ref, O.fwd_bound(x, w)) > 0


def test_zero_magnitude_requires_exact_zero():
    x = np.zeros((2, 64), np.float32)
    w = np.ones((3, 64), np.float32)
    ref = O.matmul_fwd(x, w)
    b = O.fwd_bound(x, w)
    assert O.gemm_violations(np.zeros((2, 3)), ref, b) == 0
    assert O.gemm_violations(np.full((2, 3), 1e-30), ref, b) == 6


@pytest.mark.parametrize("dq", [False, True])
def test_tiny_workload_end_to_end(dq):
    """The tiny workload through the whole oracle: shapes, sizes, bound self-consistency."""
    import synth
    t = synth.tiny()
    w = t["W"].numpy()
    q = O.quantize(w, double_quant_on=dq)
    assert q["packed"].size == 256 * 256 // 2 and q["absmax"].size == 1024
    if dq:
        assert q["absmax_q"].size == 1024 and q["scale"].size == 4
    wh = O.bf16_bits_to_f32(O.dequantize(q)).reshape(256, 256)
    x = t["X"].float().numpy()
    dy = t["dY"].float().numpy()
    y = O.matmul_fwd(x, wh)
    dx = O.matmul_bwd_dx(dy, wh)
    assert y.shape == (8, 256) and dx.shape == (8, 256)
    assert O.gemm_violations(y.astype(np.float32), y, O.fwd_bound(x, wh)) == 0
    assert O.gemm_violations(dx.astype(np.float32), dx, O.bwd_dx_bound(dy, wh)) == 0


# ------------------------------------------------------------------ adapter term (R7)
# "bitsandbytes" page, 4-bit/LoRA paragraph: frozen 4-bit base weight plus a
# trainable low-rank adapter; the layer adds (X A^T) B^T to X W^T and its input
# gradient adds (dY B) A to dY W^.

def test_lora_terms_against_exact_rationals():
    rng = np.random.default_rng(10)
    M, N, K, r = 3, 4, 64, 16
    x, w, u, b = _bf16(rng, (M, K)), _bf16(rng, (N, K), 0.02), _bf16(rng, (M, r)), _bf16(rng, (N, r), 0.1)
    dy, v, at = _bf16(rng, (M, N)), _bf16(rng, (M, r)), _bf16(rng, (K, r), 0.1)
    y = O.matmul_fwd_lora(x, w, u, b)
    dx = O.matmul_bwd_dx_lora(dy, w, v, at)
    F = lambda t: Fraction(float(t))
    for i in range(M):
        for j in range(N):
            terms = [F(x[i, k]) * F(w[j, k]) for k in range(K)] + [F(u[i, t]) * F(b[j, t]) for t in range(r)]
            assert abs(F(y[i, j]) - sum(terms)) <= Fraction(K + r) * Fraction(2) ** -52 * sum(abs(t) for t in terms)
        for k in range(K):
            terms = [F(dy[i, j]) * F(w[j, k]) for j in range(N)] + [F(v[i, t]) * F(at[k, t]) for t in range(r)]
            assert abs(F(dx[i, k]) - sum(terms)) <= Fraction(N + r) * Fraction(2) ** -52 * sum(abs(t) for t in terms)


def test_lora_special_cases():
    rng = np.random.default_rng(11)
    r, N, K = 32, 48, 128
    w, b, at = _bf16(rng, (N, K), 0.02), _bf16(rng, (N, r), 0.1), _bf16(rng, (K, r), 0.1)
    x = _bf16(rng, (r, K))
    # zero adapter activations: the plain products
    assert np.array_equal(O.matmul_fwd_lora(x, w, np.zeros((r, r)), b), O.matmul_fwd(x, w))
    # zero input, identity adapter activations: the adapter weights themselves
    eye = np.eye(r, dtype=np.float32)
    assert np.array_equal(O.matmul_fwd_lora(np.zeros((r, K)), w, eye, b), b.T.astype(np.float64))
    assert np.array_equal(O.matmul_bwd_dx_lora(np.zeros((r, N)), w, eye, at), at.T.astype(np.float64))


def test_lora_bound_rejects_mistakes():
    rng = np.random.default_rng(12)
    M, N, K, r = 8, 64, 512, 64
    x, w = _bf16(rng, (M, K)), _bf16(rng, (N, K), 0.02)
    u, b = _bf16(rng, (M, r)), _bf16(rng, (N, r), 0.1)
    ref = O.matmul_fwd_lora(x, w, u, b)
    bound = O.fwd_lora_bound(x, w, u, b)
    # fp32 accumulation in any order passes
    y32 = (x.astype(np.float32) @ w.T.astype(np.float32)) + (u.astype(np.float32) @ b.T.astype(np.float32))
    assert O.gemm_violations(y32, ref, bound) == 0
    # a dropped adapter term, a dropped base term, a sign error and a transposed operand do not
    assert O.gemm_violations(O.matmul_fwd(x, w), ref, bound) > 0
    assert O.gemm_violations(u.astype(np.float64) @ b.T, ref, bound) > 0
    assert O.gemm_violations(O.matmul_fwd(x, w) - u.astype(np.float64) @ b.T, ref, bound) > 0
    sq = _bf16(rng, (r, r), 0.1)
    assert O.gemm_violations(O.matmul_fwd(x, w)[:, :r] + u @ sq.astype(np.float64),
                             O.matmul_fwd_lora(x, w[:r], u, sq), O.fwd_lora_bound(x, w[:r], u, sq)) > 0


# ------------------------------------------------------------------ the adapter's own products (R7)

def test_adapter_products_against_exact_rationals():
    rng = np.random.default_rng(13)
    M, N, K, r, s = 3, 4, 32, 16, 0.5
    x, a = _bf16(rng, (M, K)), _bf16(rng, (r, K), 0.1)
    dy, b = _bf16(rng, (M, N)), _bf16(rng, (N, r), 0.1)
    u, v = _bf16(rng, (M, r)), _bf16(rng, (M, r))
    F = lambda t: Fraction(float(t))
    S = F(s)
    tol = lambda terms: Fraction(len(terms)) * Fraction(2) ** -52 * sum(abs(t) for t in terms)
    U, V = O.adapter_down(x, a, s), O.adapter_down_grad(dy, b, s)
    dA, dB = O.adapter_grad_down(v, x), O.adapter_grad_up(dy, u)
    for i in range(M):
        for t in range(r):
            terms = [S * F(x[i, k]) * F(a[t, k]) for k in range(K)]
            assert abs(F(U[i, t]) - sum(terms)) <= tol(terms)
            terms = [S * F(dy[i, j]) * F(b[j, t]) for j in range(N)]
            assert abs(F(V[i, t]) - sum(terms)) <= tol(terms)
    for t in range(r):
        for k in range(K):
            terms = [F(v[i, t]) * F(x[i, k]) for i in range(M)]
            assert abs(F(dA[t, k]) - sum(terms)) <= tol(terms)
    for j in range(N):
        for t in range(r):
            terms = [F(dy[i, j]) * F(u[i, t]) for i in range(M)]
            assert abs(F(dB[j, t]) - sum(terms)) <= tol(terms)


def test_adapter_gradients_are_the_derivatives_of_the_forward_term():
    """The adapter term of the forward, T(A, B) = sum(dY * ((s X A^T) B^T)), is linear in A
    and in B, so a unit change of one entry changes T by exactly that entry's gradient:
    d/dA_tk = (V^T X)_tk with V = s dY B, and d/dB_jt = (dY^T U)_jt with U = s X A^T.
    Checked in exact rationals from the forward's definition alone."""
    rng = np.random.default_rng(14)
    M, N, K, r, s = 3, 5, 6, 4, 0.25
    x, a = _bf16(rng, (M, K)), _bf16(rng, (r, K), 0.1)
    dy, b = _bf16(rng, (M, N)), _bf16(rng, (N, r), 0.1)
    F = lambda t: Fraction(float(t))
    X = [[F(x[i, k]) for k in range(K)] for i in range(M)]
    DY = [[F(dy[i, j]) for j in range(N)] for i in range(M)]

    def T(A, B):
        U = [[F(s) * sum(X[i][k] * A[t][k] for k in range(K)) for t in range(r)] for i in range(M)]
        return sum(DY[i][j] * sum(U[i][t] * B[j][t] for t in range(r)) for i in range(M) for j in range(N))

    A0 = [[F(a[t, k]) for k in range(K)] for t in range(r)]
    B0 = [[F(b[j, t]) for t in range(r)] for j in range(N)]
    base = T(A0, B0)
    V = O.adapter_down_grad(dy, b, s)
    U = O.adapter_down(x, a, s)
    dA, dB = O.adapter_grad_down(V, x), O.adapter_grad_up(dy, U)
    for t in range(r):
        for k in range(K):
            A1 = [row[:] for row in A0]
            A1[t][k] += 1
            assert abs(float(T(A1, B0) - base) - dA[t, k]) <= 1e-12 * (1 + abs(dA[t, k]))
    for j in range(N):
        for t in range(r):
            B1 = [row[:] for row in B0]
            B1[j][t] += 1
            assert abs(float(T(A0, B1) - base) - dB[j, t]) <= 1e-12 * (1 + abs(dB[j, t]))


def test_adapter_product_bound_rejects_mistakes():
    rng = np.random.default_rng(15)
    M, K, r = 64, 512, 32
    x, a = _bf16(rng, (M, K)), _bf16(rng, (r, K), 0.1)
    ref = O.adapter_down(x, a, 2.0)
    bound = O.product_bound(x, a.T, 2.0)
    # fp32 accumulation passes
    assert O.gemm_violations((x.astype(np.float32) @ a.T.astype(np.float32)) * np.float32(2.0), ref, bound) == 0
    # a missing scale and a sign error fail
    assert O.gemm_violations(ref / 2.0, ref, bound) > 0
    assert O.gemm_violations(-ref, ref, bound) > 0
    # a gradient whose reduction pairs the wrong rows (V^T against X with its rows reversed) fails
    v = _bf16(rng, (M, r))
    right = O.adapter_grad_down(v, x)
    assert O.gemm_violations(v.astype(np.float64).T @ x[::-1].astype(np.float64), right,
                             O.product_bound(v.T, x)) > 0
    # and so does dB from U with its columns reversed
    dy, u = _bf16(rng, (M, 48)), _bf16(rng, (M, r))
    assert O.gemm_violations(O.adapter_grad_up(dy, u[:, ::-1]), O.adapter_grad_up(dy, u),
                             O.product_bound(dy.T, u)) > 0
