"""GPU parity: the fused NF4-dequant GEMMs against the CPU oracle.

Forward Y = X W^T and backward dX = dY W^ ("Zenbit" page, zenbit.pallas_nf4
bullet: fused forward and a fused backward forming dL/dX only).  The oracle
quantizes the same seeded weight itself, rounds W^ to bf16 the same way and
accumulates in float64; every output element, at every workload size, must
satisfy |err| <= 1e-4 * (|A| |B|) (1e-4 is the stated tolerance).
Identity inputs make the product a copy of W^, which must then be exact.
"""
import numpy as np
import pytest
import torch

import oracle as O
import synth
from tests._gpu import assert_gemm_rows, assert_gemm_within_bound, bf16_bits, dev, lib, note, oracle_quantize

pytestmark = pytest.mark.gpu


def _oracle_what(W_cpu, dq=True):
    qo = oracle_quantize(W_cpu, dq)
    return O.bf16_bits_to_f32(O.dequantize(qo)).reshape(W_cpu.shape)


def _run(M, N, K, seed, dq=True, out_dtype=torch.float32, wdtype=torch.bfloat16):
    dg = lib()
    d = dev()
    W = synth.normal((N, K), 0.02, seed, wdtype)
    X = synth.normal((M, K), 1.0, seed + 1)
    dY = synth.normal((M, N), 1.0, seed + 2)
    q = dg.nf4_quantize(W.to(d), double_quant=dq)
    Y = dg.nf4_matmul_fwd(X.to(d), q, out_dtype)
    dX = dg.nf4_matmul_bwd_dx(dY.to(d), q, out_dtype)
    torch.cuda.synchronize()
    wh = _oracle_what(W, dq)
    x = X.float().numpy()
    dy = dY.float().numpy()
    return Y, dX, x, dy, wh


@pytest.mark.parametrize("M,N,K", [
    (1, 256, 256), (4, 256, 256), (8, 256, 256), (16, 256, 256),    # small-M kernel
    (1, 300, 320), (5, 17, 64), (16, 1000, 192), (3, 4096, 4096),
    (16, 200, 4096), (2, 64, 8192), (1, 48, 40960),                  # small-M: X from global, many K chunks
    (17, 300, 256), (100, 513, 128), (256, 256, 256), (300, 700, 512),  # large-M kernel, ragged tiles
    (513, 129, 64), (1000, 64, 1024), (400, 260, 192), (769, 384, 320),
])
def test_fwd_bwd_ragged(M, N, K):
    Y, dX, x, dy, wh = _run(M, N, K, 7 * M + N + K)
    assert_gemm_within_bound(Y, O.matmul_fwd(x, wh), O.fwd_bound(x, wh), f"fwd {M}x{N}x{K}")
    assert_gemm_within_bound(dX, O.matmul_bwd_dx(dy, wh), O.bwd_dx_bound(dy, wh), f"bwd {M}x{N}x{K}")


@pytest.mark.parametrize("dq", [True, False])
def test_tiny_workload(dq):
    dg = lib()
    d = dev()
    t = synth.tiny()
    q = dg.nf4_quantize(t["W"].to(d), double_quant=dq)
    Y = dg.nf4_matmul_fwd(t["X"].to(d), q)
    dX = dg.nf4_matmul_bwd_dx(t["dY"].to(d), q)
    torch.cuda.synchronize()
    wh = _oracle_what(t["W"], dq)
    x, dy = t["X"].float().numpy(), t["dY"].float().numpy()
    assert_gemm_within_bound(Y, O.matmul_fwd(x, wh), O.fwd_bound(x, wh), "tiny fwd")
    assert_gemm_within_bound(dX, O.matmul_bwd_dx(dy, wh), O.bwd_dx_bound(dy, wh), "tiny bwd")


@pytest.mark.parametrize("n_rows,k_cols", [(256, 256), (320, 192)])
def test_identity_inputs_reproduce_the_dequantized_weight(n_rows, k_cols):
    """X = I gives Y = W^T, dY = I gives dX = W^: each output is one exact product."""
    dg = lib()
    d = dev()
    W = synth.tiny()["W"] if (n_rows, k_cols) == (256, 256) else synth.normal((n_rows, k_cols), 0.02, 77, torch.float32)
    wh = _oracle_what(W)
    q = dg.nf4_quantize(W.to(d), double_quant=True)
    for M in (k_cols,):
        Y = dg.nf4_matmul_fwd(torch.eye(k_cols, dtype=torch.bfloat16, device=d), q)
        assert np.array_equal(Y.cpu().numpy(), wh.T)
    dX = dg.nf4_matmul_bwd_dx(torch.eye(n_rows, dtype=torch.bfloat16, device=d), q)
    assert np.array_equal(dX.cpu().numpy(), wh)
    # small-M kernel: unit rows pick single columns of W^
    e = torch.zeros((4, k_cols), dtype=torch.bfloat16)
    for r, kk in enumerate((0, 1, 63, k_cols - 1)):
        e[r, kk] = 1
    Ys = dg.nf4_matmul_fwd(e.to(d), q)
    torch.cuda.synchronize()
    assert np.array_equal(Ys.cpu().numpy(), wh[:, [0, 1, 63, k_cols - 1]].T)


def test_bf16_outputs_are_one_rounding_of_fp32():
    dg = lib()
    d = dev()
    W = synth.normal((384, 512), 0.02, 3, torch.bfloat16).to(d)
    q = dg.nf4_quantize(W)
    for M in (8, 300):
        X = synth.normal((M, 512), 1.0, 4).to(d)
        dY = synth.normal((M, 384), 1.0, 5).to(d)
        y32 = dg.nf4_matmul_fwd(X, q, torch.float32)
        y16 = dg.nf4_matmul_fwd(X, q, torch.bfloat16)
        d32 = dg.nf4_matmul_bwd_dx(dY, q, torch.float32)
        d16 = dg.nf4_matmul_bwd_dx(dY, q, torch.bfloat16)
        torch.cuda.synchronize()
        assert np.array_equal(bf16_bits(y16), O.f32_to_bf16_bits(y32.cpu().numpy()))
        assert np.array_equal(bf16_bits(d16), O.f32_to_bf16_bits(d32.cpu().numpy()))


def test_zero_rows_is_a_noop():
    dg = lib()
    d = dev()
    q = dg.nf4_quantize(synth.normal((64, 64), 0.02, 1).to(d))
    Y = dg.nf4_matmul_fwd(torch.empty((0, 64), dtype=torch.bfloat16, device=d), q)
    dX = dg.nf4_matmul_bwd_dx(torch.empty((0, 64), dtype=torch.bfloat16, device=d), q)
    assert Y.shape == (0, 64) and dX.shape == (0, 64)


def test_deterministic_reruns():
    dg = lib()
    d = dev()
    q = dg.nf4_quantize(synth.normal((1024, 1024), 0.02, 8).to(d))
    for M in (4, 512):
        X = synth.normal((M, 1024), 1.0, 9).to(d)
        a = dg.nf4_matmul_fwd(X, q)
        b = dg.nf4_matmul_fwd(X, q)
        c = dg.nf4_matmul_bwd_dx(X, q)
        e = dg.nf4_matmul_bwd_dx(X, q)
        torch.cuda.synchronize()
        assert torch.equal(a, b) and torch.equal(c, e)


@pytest.mark.parametrize("M", synth.DECODE_MS)
def test_decode_full(M):
    dg = lib()
    d = dev()
    W = synth.decode_weight(0)
    X = synth.decode_x(M)
    q = dg.nf4_quantize(W.to(d))
    Y = dg.nf4_matmul_fwd(X.to(d), q)
    torch.cuda.synchronize()
    wh = _oracle_what(W)
    x = X.float().numpy()
    assert_gemm_within_bound(Y, O.matmul_fwd(x, wh), O.fwd_bound(x, wh), f"decode M={M}")


@pytest.mark.parametrize("N,K", [(1000, 2048), (520, 4096)])
def test_small_m_every_row_count(N, K):
    """M = 1 .. 16 on one weight: the small-M forward reads X per lane below 11 rows and from
    the copy staged in LDS from 11 rows on; K = 2048 puts two rows of X in one copy round of
    the eight waves (a wave's first piece in the second row), K = 4096 one."""
    dg = lib()
    d = dev()
    W = synth.normal((N, K), 0.02, 7 * N + K, torch.bfloat16)
    q = dg.nf4_quantize(W.to(d))
    wh = _oracle_what(W).astype(np.float64)
    for M in range(1, 17):
        note(f"small-M fwd M={M} N={N} K={K}")
        X = synth.normal((M, K), 1.0, 100 * M + K)
        Y = dg.nf4_matmul_fwd(X.to(d), q)
        torch.cuda.synchronize()
        x = X.float().numpy()
        assert_gemm_within_bound(Y, O.matmul_fwd(x, wh), O.fwd_bound(x, wh), f"small M={M} N={N} K={K}")


@pytest.mark.parametrize("N,K", [(1000, 2048), (8, 64), (4104, 192)])
def test_small_m_backward_every_row_count(N, K):
    """M = 1 .. 16 rows of dY on one weight: the small-M backward (one workgroup per 64 output
    columns, 64-row steps over N dealt to 16 waves); N = 1000 and 4104 end in a partial step and
    leave some waves without a step, N = 8 is a single partial step, K = 64 a single workgroup."""
    dg = lib()
    d = dev()
    W = synth.normal((N, K), 0.02, 3 * N + K, torch.bfloat16)
    q = dg.nf4_quantize(W.to(d))
    wh = _oracle_what(W).astype(np.float64)
    for M in range(1, 17):
        note(f"small-M bwd M={M} N={N} K={K}")
        dY = synth.normal((M, N), 1.0, 200 * M + N)
        dYd = dY.to(d)
        dX = dg.nf4_matmul_bwd_dx(dYd, q)
        dX16 = dg.nf4_matmul_bwd_dx(dYd, q, torch.bfloat16)
        again = dg.nf4_matmul_bwd_dx(dYd, q)
        torch.cuda.synchronize()
        assert torch.equal(dX, again), "deterministic"
        assert np.array_equal(bf16_bits(dX16), O.f32_to_bf16_bits(dX.cpu().numpy()))
        dy = dY.float().numpy()
        assert_gemm_within_bound(dX, O.matmul_bwd_dx(dy, wh), O.bwd_dx_bound(dy, wh), f"small bwd M={M} N={N} K={K}")


@pytest.mark.parametrize("M,N,K", [(17, 1000, 2048), (33, 520, 4096), (100, 1000, 2048), (224, 264, 4096),
                                   (40, 4104, 11008)])
def test_small_m_backward_grid_rows(M, N, K):
    """Above 16 rows of dY the small-M backward gives each 16 rows a grid row of their own while
    its estimated time stays below the 256x256 kernel's (a last grid row of one row at 17 and
    33, 64-column bands at K = 11008); every element against the oracle, bf16 the one rounding
    of fp32, reruns bitwise identical."""
    note(f"small-M bwd grid rows M={M} N={N} K={K}")
    dg = lib()
    d = dev()
    W = synth.normal((N, K), 0.02, 5 * M + N, torch.bfloat16)
    dY = synth.normal((M, N), 1.0, 7 * M + K)
    q = dg.nf4_quantize(W.to(d))
    dYd = dY.to(d)
    dX = dg.nf4_matmul_bwd_dx(dYd, q)
    dX16 = dg.nf4_matmul_bwd_dx(dYd, q, torch.bfloat16)
    again = dg.nf4_matmul_bwd_dx(dYd, q)
    torch.cuda.synchronize()
    assert torch.equal(dX, again)
    assert np.array_equal(bf16_bits(dX16), O.f32_to_bf16_bits(dX.cpu().numpy()))
    wh = _oracle_what(W).astype(np.float64)
    dy = dY.float().numpy()
    assert_gemm_within_bound(dX, O.matmul_bwd_dx(dy, wh), O.bwd_dx_bound(dy, wh), f"grid rows bwd M={M} N={N} K={K}")


@pytest.fixture(scope="module")
def prefill():
    dg = lib()
    d = dev()
    note("prefill: drawing inputs, GPU quantize/fwd/bwd")
    W = synth.prefill_weight()
    X, dY = synth.prefill_x(), synth.prefill_dy()
    q = dg.nf4_quantize(W.to(d))
    Y = dg.nf4_matmul_fwd(X.to(d), q)
    dX = dg.nf4_matmul_bwd_dx(dY.to(d), q)
    torch.cuda.synchronize()
    note("prefill: oracle W^")
    return {"X": X, "dY": dY, "Y": Y.cpu(), "dX": dX.cpu(), "wh": _oracle_what(W).astype(np.float64)}


def test_prefill_fwd_every_element(prefill):
    """All 4096 x 11008 outputs of Y = X W^T against the oracle's float64 product."""
    assert_gemm_rows(prefill["Y"], prefill["X"], prefill["wh"], "fwd", "prefill fwd")


def test_prefill_bwd_every_element(prefill):
    """All 4096 x 4096 outputs of dX = dY W^ (reduction over 11008) against the oracle."""
    assert_gemm_rows(prefill["dX"], prefill["dY"], prefill["wh"], "bwd_dx", "prefill bwd")


@pytest.fixture(scope="module")
def large(large_oracle):
    dg = lib()
    d = dev()
    W, qo = large_oracle
    note("large: drawing X and dY; GPU quantize/fwd/bwd")
    X, dY = synth.large_x(), synth.large_dy()
    q = dg.nf4_quantize(W.to(d))
    Y = dg.nf4_matmul_fwd(X.to(d), q)
    dX = dg.nf4_matmul_bwd_dx(dY.to(d), q)
    # decode on the same weight: the first M rows of X
    dec = {M: dg.nf4_matmul_fwd(X[:M].to(d), q) for M in synth.DECODE_MS}
    torch.cuda.synchronize()
    out = {"X": X, "dY": dY, "Y": Y.cpu(), "dX": dX.cpu(), "dec": {M: y.cpu() for M, y in dec.items()}}
    del Y, dX, q, dec
    torch.cuda.empty_cache()
    note("large: oracle W^ (235M elements)")
    out["wh"] = O.bf16_bits_to_f32(O.dequantize(qo)).reshape(W.shape).astype(np.float64)
    return out


def test_large_fwd_every_element(large):
    """All 8192 x 28672 outputs of the outlier-heavy forward against the oracle."""
    assert_gemm_rows(large["Y"], large["X"], large["wh"], "fwd", "large fwd")


def test_large_bwd_every_element(large):
    """All 8192 x 8192 outputs of dX (reduction over 28672) against the oracle."""
    assert_gemm_rows(large["dX"], large["dY"], large["wh"], "bwd_dx", "large bwd")


def test_large_decode_every_element(large):
    """Decode (M = 1, 4, 16) on the 28672 x 8192 weight: all outputs against the oracle."""
    for M, y in large["dec"].items():
        x = large["X"][:M].float().numpy()
        assert_gemm_within_bound(y, O.matmul_fwd(x, large["wh"]), O.fwd_bound(x, large["wh"]), f"large decode M={M}")
