"""Shared helpers of the GPU parity tests: device checks and oracle comparisons.

Expected values always come from ``oracle`` run on the same seeded inputs;
nothing here derives an expected value from the HIP path.
"""
import sys

import numpy as np
import pytest
import torch

import oracle as O


def dev():
    if not torch.cuda.is_available():
        pytest.fail("GPU test run without a HIP device")
    return torch.device("cuda:0")


def lib():
    import dequant_gemm_amd as dg
    dg.lib()  # raises if libnf4.so is missing: no fallback
    return dg


CONFIG = None   # the pytest config, set by conftest.py


def note(msg: str):
    """Progress line written past pytest's output capture (it names the case before a GPU step)."""
    capman = CONFIG.pluginmanager.getplugin("capturemanager") if CONFIG is not None else None
    if capman is None:
        sys.__stderr__.write(msg + "\n")
        sys.__stderr__.flush()
        return
    with capman.global_and_fixture_disabled():
        sys.stderr.write(msg + "\n")
        sys.stderr.flush()


def u32(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().view(torch.int32).numpy().view(np.uint32)


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def oracle_quantize(w_cpu: torch.Tensor, dq: bool) -> dict:
    return O.quantize(w_cpu.float().numpy(), double_quant_on=dq)


def assert_quant_equal(qg, qo: dict, where: str = ""):
    """Codes (packed bytes) and the absmax state, bit for bit."""
    pk = qg.packed.cpu().numpy()
    bad = np.nonzero(pk != qo["packed"])[0]
    assert bad.size == 0, f"{where}: {bad.size} packed bytes differ, first at {bad[0]}"
    if qo["double_quant"]:
        assert u32(qg.absmax_mean)[0] == np.float32(qo["mean"]).view(np.uint32), f"{where}: mean"
        q = qg.absmax_q.cpu().numpy()
        bad = np.nonzero(q != qo["absmax_q"])[0]
        assert bad.size == 0, f"{where}: {bad.size} int8 absmax differ, first at {bad[0]}"
        s = u32(qg.absmax_scale)
        assert np.array_equal(s, qo["scale"].view(np.uint32)), f"{where}: scales"
    else:
        a = u32(qg.absmax)
        bad = np.nonzero(a != qo["absmax"].view(np.uint32))[0]
        assert bad.size == 0, f"{where}: {bad.size} fp32 absmax differ, first at {bad[0]}"


def assert_gemm_within_bound(out: torch.Tensor, ref: np.ndarray, bound: np.ndarray, where: str = ""):
    o = out.detach().float().cpu().numpy().astype(np.float64)
    assert o.shape == ref.shape
    assert np.all(np.isfinite(o)), f"{where}: non-finite output"
    err = np.abs(o - ref)
    bad = ~(err <= bound)
    n = int(bad.sum())
    if n:
        i = np.argwhere(bad)[0]
        pytest.fail(f"{where}: {n} elements outside 1e-4*(|A||B|); first {tuple(i)}: "
                    f"got {o[tuple(i)]!r} want {ref[tuple(i)]!r} bound {bound[tuple(i)]!r}")


def assert_gemm_rows(out: torch.Tensor, a_bf16: torch.Tensor, wh64: np.ndarray, op: str, where: str,
                     rows: int = 1024):
    """Every element of a GEMM output against the oracle, in chunks of ``rows`` output rows.

    ``out`` is the GPU result (any device), ``a_bf16`` the left operand (X for the
    forward, dY for the backward) on the host, ``wh64`` the oracle's W^ as float64.
    Each chunk takes the oracle's float64 product and its element-wise bound.
    """
    if op == "fwd":
        prod, bound = O.matmul_fwd, O.fwd_bound
    elif op == "bwd_dx":
        prod, bound = O.matmul_bwd_dx, O.bwd_dx_bound
    else:
        raise ValueError(op)
    out = out.detach().cpu()
    M = a_bf16.shape[0]
    assert out.shape[0] == M
    for lo in range(0, M, rows):
        hi = min(M, lo + rows)
        a = a_bf16[lo:hi].float().numpy()
        assert_gemm_within_bound(out[lo:hi], prod(a, wh64), bound(a, wh64), f"{where} rows {lo}..{hi - 1}")
        note(f"{where}: rows {lo}..{hi - 1} of {M} within the bound")

