"""The C ABI on the CPU: the library loads, exports every call include/nf4.h
declares, its constants agree with the oracle, sizes follow the closed forms,
and every host-detectable error is returned before any HIP call.

No compute call is made here (no GPU); the error paths never reach HIP.
"""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

import oracle as O
from tests._exact import exact_argmin_code

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "nf4.h")

dg = pytest.importorskip("dequant_gemm_amd")


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(dg.LIB_PATH):
        pytest.fail("libnf4.so is not built (run `python -m dequant_gemm_amd.build`)")
    return dg.lib()


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(nf4_[a-z0-9_]+)\s*\(", text)))


def test_every_declared_function_is_exported(L):
    declared = _declared_functions()
    assert set(declared) == set(dg.EXPORTS)
    out = subprocess.run(["nm", "-D", "--defined-only", dg.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (nf4_[a-z0-9_]+)$", out, flags=re.M))
    assert set(declared) <= exported, set(declared) - exported
    for name in declared:
        assert hasattr(L, name)


def test_codebook_matches_oracle_bit_for_bit(L):
    got = dg.nf4_codebook().numpy()
    assert got.view(np.uint32).tolist() == O.codebook().view(np.uint32).tolist()


def test_levels_of_both_types_match_oracle_bit_for_bit(L):
    for qt, want in (("nf4", O.codebook()), ("fp4", O.fp4_codebook())):
        got = dg.nf4_levels(qt).numpy()
        assert got.view(np.uint32).tolist() == want.view(np.uint32).tolist(), qt
    out = (ctypes.c_float * 16)()
    assert L.nf4_levels(2, out) == 9 and L.nf4_levels(-1, out) == 9
    assert L.nf4_levels(0, None) == 1


def test_qtensor_struct_layout():
    """quant_type is the last field: the earlier fields keep their offsets."""
    S = dg.QTensorStruct
    assert (S.rows.offset, S.cols.offset, S.blocksize.offset, S.double_quant.offset, S.packed.offset) == (0, 8, 16, 20, 24)
    assert (S.absmax_mean.offset, S.quant_type.offset, ctypes.sizeof(S)) == (56, 64, 72)
    assert _qt().quant_type == 0 and dg.QTensorStruct(1, 1, 64, 0).quant_type == 0   # zero tail = NF4


def test_quant_type_is_checked_by_every_call(L):
    ws = dg.nf4_sizes(64, 64, 64, True)["workspace_bytes"]
    for bad in (2, -1, 7):
        q = _qt(qt=bad)
        assert L.nf4_quantize(P, 1, 64, 64, 64, 1, ctypes.byref(q), P, ws, None, None) == 9
        assert L.nf4_dequantize(ctypes.byref(q), P, 1, None) == 9
        assert L.nf4_matmul_fwd(P, 4, ctypes.byref(q), P, 0, None) == 9
        assert L.nf4_matmul_bwd_dx(P, 4, ctypes.byref(q), P, 0, None) == 9
    with pytest.raises(ValueError):
        dg.empty_qtensor(4, 64, True, "cpu", 64, "int4")


def test_thresholds_are_the_exact_decision_boundaries(L):
    """Each t_i is the smallest fp32 whose exact nearest level is i+1 (ties to the lower)."""
    c = O.codebook()
    t = dg.nf4_thresholds().numpy()
    assert np.all(np.diff(t.astype(np.float64)) > 0)
    for i, ti in enumerate(t):
        below = np.nextafter(np.float32(ti), np.float32(-2))
        assert exact_argmin_code(np.float32(ti), c) == i + 1
        assert exact_argmin_code(below, c) == i


@pytest.mark.parametrize("bs", [32, 64, 128, 256])
@pytest.mark.parametrize("rows,cols,dq", [(256, 256, True), (4096, 4096, True), (11008, 4096, True),
                                          (28672, 8192, True), (3, 37, False), (1, 1, True)])
def test_sizes_closed_forms(L, rows, cols, dq, bs):
    s = dg.nf4_sizes(rows, cols, bs, dq)
    numel = rows * cols
    nb = -(-numel // bs)
    assert s["packed_bytes"] == -(-numel // 2)
    assert s["nblocks"] == nb
    assert s["ngroups"] == -(-nb // 256)
    if dq:
        assert s["workspace_bytes"] >= 512 * 128 + 4 * nb
    else:
        assert s["workspace_bytes"] == 0


def test_appendix_quantized_bytes():
    """Wq = packed + int8 absmax + fp32 scales + mu at the workload sizes (4.127 bits/weight)."""
    expect = {(256, 256): 33812, (4096, 4096): 8654852, (11008, 4096): 23259908, (28672, 8192): 121167876}
    for (r, c), wq in expect.items():
        s = dg.nf4_sizes(r, c, 64, True)
        assert s["packed_bytes"] + s["nblocks"] + 4 * s["ngroups"] + 4 == wq


def _status(name, L):
    return getattr(dg._lib, "NF4_" + name) if hasattr(dg._lib, "NF4_" + name) else None


P = 1 << 20  # a fake, 16-byte aligned "device" address; never dereferenced on the error paths


def _qt(rows=64, cols=64, dq=1, packed=P, absmax=P, q=P, scale=P, mean=P, bs=64, qt=0):
    return dg.QTensorStruct(rows, cols, bs, dq, packed, absmax, q, scale, mean, qt)


def test_sizes_errors(L):
    i64 = ctypes.c_int64
    assert L.nf4_sizes(0, 64, 64, 1, None, None, None, None) == 2
    assert L.nf4_sizes(64, -1, 64, 1, None, None, None, None) == 2
    assert L.nf4_sizes(1 << 20, 1 << 20, 64, 1, None, None, None, None) == 2  # beyond 2^36 elements
    # exactly 2^36 elements is accepted at every block size (the block count stays below 2^31);
    # one more row is not
    nb = i64()
    for bs in (32, 64, 128, 256):
        assert L.nf4_sizes(1 << 18, 1 << 18, bs, 1, None, ctypes.byref(nb), None, None) == 0
        assert nb.value == (1 << 36) // bs
        assert L.nf4_sizes((1 << 18) + 1, 1 << 18, bs, 1, None, None, None, None) == 2
    for bs in (0, 16, 48, 96, 512, -64):                  # block sizes: 32, 64, 128 or 256
        assert L.nf4_sizes(64, 64, bs, 1, None, None, None, None) == 3
    assert L.nf4_sizes(64, 64, 64, 2, None, None, None, None) == 7
    assert L.nf4_codebook(None) == 1


def test_quantize_errors(L):
    q = _qt()
    ws = dg.nf4_sizes(64, 64, 64, True)["workspace_bytes"]
    call = lambda **k: L.nf4_quantize(k.get("W", P), k.get("dt", 1), k.get("rows", 64), k.get("cols", 64),
                                      k.get("bs", 64), k.get("dq", 1), ctypes.byref(k.get("q", q)),
                                      k.get("ws", P), k.get("wsb", ws), k.get("status", None), None)
    assert call(W=None) == 1
    assert call(dt=7) == 4
    assert call(bs=48) == 3
    assert call(bs=128) == 2                         # descriptor's block size (64) differs from the call's
    assert call(rows=0) == 2
    assert call(W=P + 2) == 5
    assert call(wsb=ws - 1) == 6
    assert call(ws=None) == 1
    assert call(ws=P + 8) == 5
    assert call(q=_qt(rows=32)) == 2                 # descriptor does not match the shape
    assert call(q=_qt(dq=0), dq=1) == 2
    assert call(q=_qt(packed=None)) == 1
    assert call(q=_qt(q=None)) == 1
    assert call(q=_qt(mean=P + 4)) == 5
    assert call(status=P + 4) == 5
    assert L.nf4_quantize(P, 1, 64, 64, 64, 1, None, P, ws, None, None) == 1


def test_quantize_noalloc_errors(L):
    """The allocation-free quantize checks as nf4_quantize does, and refuses a tensor with
    more blocks than its fixed scratch holds, all before any HIP call."""
    q = _qt()
    call = lambda **k: L.nf4_quantize_noalloc(k.get("W", P), k.get("dt", 1), k.get("rows", 64),
                                              k.get("cols", 64), k.get("bs", 64), k.get("dq", 1),
                                              ctypes.byref(k.get("q", q)), k.get("status", None), None)
    assert call(W=None) == 1
    assert call(dt=7) == 4
    assert call(bs=48) == 3
    assert call(rows=0) == 2
    assert call(W=P + 2) == 5
    assert call(q=_qt(rows=32)) == 2
    assert call(q=_qt(q=None)) == 1
    assert call(status=P + 4) == 5
    assert L.nf4_quantize_noalloc(P, 1, 64, 64, 64, 1, None, None, None) == 1
    # the scratch limit: NF4_NOALLOC_MAX_BLOCKS blocks with double quantization
    limit = dg.NOALLOC_MAX_BLOCKS
    header = open(HEADER).read()
    assert re.search(r"#define NF4_NOALLOC_MAX_BLOCKS \(\(int64_t\)1 << 22\)", header)
    for bs in (32, 64, 256):
        rows, cols = limit * bs // 4096 + 1, 4096          # limit + 4096 / bs blocks
        assert call(rows=rows, cols=cols, bs=bs, q=_qt(rows=rows, cols=cols, bs=bs)) == 10


def test_dequantize_errors(L):
    assert L.nf4_dequantize(None, P, 1, None) == 1
    assert L.nf4_dequantize(ctypes.byref(_qt()), None, 1, None) == 1
    assert L.nf4_dequantize(ctypes.byref(_qt()), P, 5, None) == 4
    assert L.nf4_dequantize(ctypes.byref(_qt()), P + 2, 1, None) == 5
    assert L.nf4_dequantize(ctypes.byref(_qt(bs=16)), P, 1, None) == 3
    assert L.nf4_dequantize(ctypes.byref(_qt(dq=0, absmax=None)), P, 1, None) == 1


@pytest.mark.parametrize("fn", ["nf4_matmul_fwd", "nf4_matmul_bwd_dx"])
def test_gemm_errors(L, fn):
    f = getattr(L, fn)
    q = _qt(rows=128, cols=256)
    assert f(P, 4, None, P, 0, None) == 1
    assert f(None, 4, ctypes.byref(q), P, 0, None) == 1
    assert f(P, 4, ctypes.byref(q), None, 0, None) == 1
    assert f(P, -1, ctypes.byref(q), P, 0, None) == 2
    assert f(P, 4, ctypes.byref(q), P, 9, None) == 4
    assert f(P + 4, 4, ctypes.byref(q), P, 0, None) == 5
    assert f(P, 4, ctypes.byref(_qt(rows=128, cols=96)), P, 0, None) == 7   # K % 64 != 0
    assert f(P, 4, ctypes.byref(_qt(rows=1, cols=1 << 24)), P, 0, None) == 7   # K at the column limit
    # M == 0 is a successful no-op that launches nothing
    assert f(None, 0, ctypes.byref(q), None, 0, None) == 0


def test_status_strings(L):
    for s in range(11):
        assert L.nf4_status_string(s)
    assert L.nf4_status_string(99) == b"unknown status"


@pytest.mark.parametrize("fn", ["nf4_matmul_fwd_lora", "nf4_matmul_bwd_dx_lora"])
def test_lowrank_gemm_errors(L, fn):
    f = getattr(L, fn)
    q = _qt(rows=128, cols=256)
    ok = lambda **k: f(k.get("A", P), k.get("M", 4), ctypes.byref(k.get("q", q)), k.get("U", P), k.get("V", P),
                       k.get("r", 16), k.get("C", P), k.get("dt", 0), None)
    assert ok(A=None) == 1
    assert ok(C=None) == 1
    assert ok(U=None) == 1
    assert ok(V=None) == 1
    assert ok(U=P + 8) == 5
    assert ok(V=P + 2) == 5
    for r in (0, 8, 24, 1040, -16):
        assert ok(r=r) == 7                                 # rank: multiple of 16 in [16, 1024]
    assert ok(q=_qt(rows=128, cols=96)) == 7               # K % 64 != 0, as without the adapter
    assert ok(dt=3) == 4
    assert f(P, 4, None, P, P, 16, P, 0, None) == 1
    # M == 0: a successful no-op once the rank is valid
    assert f(None, 0, ctypes.byref(q), None, None, 32, None, 0, None) == 0
    assert f(None, 0, ctypes.byref(q), None, None, 17, None, 0, None) == 7


def test_bench_stream_library_exports_and_refuses_bad_arguments():
    """libnf4_bench (include/nf4_bench.h): every declared call is exported, and every bad
    argument is refused with status 1 before anything is launched."""
    from dequant_gemm_amd.build import BENCH_LIB
    if not os.path.exists(BENCH_LIB):
        pytest.fail("libnf4_bench.so is not built (run `python -m dequant_gemm_amd.build`)")
    text = re.sub(r"/\*.*?\*/", "", open(os.path.join(ROOT, "include", "nf4_bench.h")).read(), flags=re.S)
    declared = set(re.findall(r"\b(nf4bench_[a-z0-9_]+)\s*\(", text))
    out = subprocess.run(["nm", "-D", "--defined-only", BENCH_LIB], capture_output=True, text=True).stdout
    assert declared and declared <= set(re.findall(r"\bT (nf4bench_[a-z0-9_]+)$", out, flags=re.M))
    B = ctypes.CDLL(BENCH_LIB)
    f = B.nf4bench_read_stream
    f.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    f.restype = ctypes.c_int
    assert f(None, 1 << 20, P, 256, 256, None) == 1
    assert f(P, 1 << 20, None, 256, 256, None) == 1
    assert f(P, 0, P, 256, 256, None) == 1
    assert f(P, (1 << 20) + 8, P, 256, 256, None) == 1     # not a multiple of 16
    assert f(P + 4, 1 << 20, P, 256, 256, None) == 1        # misaligned source
    assert f(P, 1 << 20, P + 4, 256, 256, None) == 1        # misaligned sink
    assert f(P, 1 << 20, P, 256, 100, None) == 1            # block size
    assert f(P, 1 << 20, P, 0, 256, None) == 1              # grid
    assert f(P, 1 << 20, P, 65537, 256, None) == 1
