"""GPU parity: nf4_quantize and nf4_dequantize against the CPU oracle, bit for bit.

Codes, packed bytes, fp32/int8 absmax, scales, mean and dequantized weights
must equal the oracle's exactly ("Zenbit" page, zenbit.nf4 bullet;
"bitsandbytes" page, NF4 and double-quantization paragraphs).
"""
import concurrent.futures as cf
import os

import numpy as np
import pytest
import torch

import oracle as O
import synth
from tests._gpu import assert_quant_equal, bf16_bits, dev, lib, note, oracle_quantize, u32

pytestmark = pytest.mark.gpu


def _check_roundtrip(W_cpu, dq, where):
    dg = lib()
    d = dev()
    qo = oracle_quantize(W_cpu, dq)
    qg = dg.nf4_quantize(W_cpu.to(d), double_quant=dq)
    torch.cuda.synchronize()
    assert_quant_equal(qg, qo, where)
    wh = dg.nf4_dequantize(qg, torch.bfloat16)
    want = O.dequantize(qo).reshape(W_cpu.shape)
    got = bf16_bits(wh)
    bad = np.nonzero(got != want)
    assert bad[0].size == 0, f"{where}: {bad[0].size} bf16 W^ differ"
    wf = dg.nf4_dequantize(qg, torch.float32)
    assert np.array_equal(u32(wf), O.dequantize(qo, out="f32").reshape(W_cpu.shape).view(np.uint32)), where
    return qg, qo


@pytest.mark.parametrize("dq", [True, False])
def test_tiny(dq):
    _check_roundtrip(synth.tiny()["W"], dq, f"tiny dq={dq}")


@pytest.mark.parametrize("rows,cols", [(1, 1), (1, 2), (3, 37), (5, 64), (1, 100), (7, 1000),
                                       (33, 65), (2, 8191), (300, 777), (257, 256 * 64 + 8)])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_ragged_shapes(rows, cols, dtype):
    W = synth.normal((rows, cols), 0.02, 17 + rows + cols, dtype)
    for dq in (True, False):
        _check_roundtrip(W, dq, f"{rows}x{cols} {dtype} dq={dq}")


def _special_weight():
    """Blocks that exercise every branch of the level search."""
    rng = np.random.default_rng(99)
    c = O.codebook()
    blocks = []
    blocks.append(np.zeros(64, np.float32))                                            # all zero
    blocks.append((rng.standard_normal(64) * 1e-40).astype(np.float32))               # subnormal
    blocks.append((rng.uniform(-1, 1, 64) * 2.0 ** -126).astype(np.float32))          # tiny normal
    blocks.append((rng.uniform(-1, 1, 64) * 3.0e38).astype(np.float32))               # near overflow
    # exact ties: absmax 1.0, so n = x exactly; the five exactly representable midpoints
    mids = [(np.float64(c[i]) + np.float64(c[i + 1])) / 2 for i in range(15)]
    exact = [np.float32(m) for m in mids if float(np.float32(m)) == m]
    b = np.zeros(64, np.float32)
    b[0] = 1.0
    vals = []
    for m in exact:
        vals += [m, np.nextafter(m, np.float32(2)), np.nextafter(m, np.float32(-2))]
    for m in mids:  # values within an ulp of every threshold
        f = np.float32(m)
        vals += [f, np.nextafter(f, np.float32(2)), np.nextafter(f, np.float32(-2))]
    b[1:1 + min(63, len(vals))] = np.array(vals[:63], np.float32)
    blocks.append(b)
    b2 = b.copy()
    b2[0] = -1.0
    b2[1:] = -b2[1:]
    blocks.append(b2)
    rest = vals[63:]
    b3 = np.zeros(64, np.float32)
    b3[0] = 1.0
    b3[1:1 + len(rest)] = np.array(rest[:63], np.float32)
    blocks.append(b3)
    # the same patterns scaled by an absmax that is not a power of two
    s = np.float32(0.0371)
    blocks.append((b * s).astype(np.float32))
    blocks.append(np.full(64, np.float32(-0.5)))                                      # constant block
    blocks.append((rng.standard_normal(64) * 0.02).astype(np.float32))
    w = np.concatenate(blocks).reshape(-1, 64)
    return torch.from_numpy(w)


@pytest.mark.parametrize("dq", [True, False])
def test_special_blocks(dq):
    _check_roundtrip(_special_weight(), dq, f"special dq={dq}")


def test_nonfinite_input_sets_status_bit():
    dg = lib()
    d = dev()
    W = synth.normal((4, 256), 0.02, 5, torch.float32)
    W[2, 70] = float("inf")
    status = torch.zeros(4, dtype=torch.int32, device=d)
    dg.nf4_quantize(W.to(d), double_quant=True, status=status)
    torch.cuda.synchronize()
    assert int(status[0].item()) & 1 == 1
    status.zero_()
    dg.nf4_quantize(synth.normal((4, 256), 0.02, 5, torch.float32).to(d), double_quant=True, status=status)
    torch.cuda.synchronize()
    assert int(status[0].item()) == 0


def test_deterministic_and_mean_is_order_free():
    dg = lib()
    d = dev()
    W = synth.normal((2048, 512), 0.02, 41, torch.bfloat16).to(d)
    a = dg.nf4_quantize(W)
    b = dg.nf4_quantize(W)
    torch.cuda.synchronize()
    for name in ("packed", "absmax_q", "absmax_scale", "absmax_mean"):
        assert torch.equal(getattr(a, name), getattr(b, name)), name
    # permuting rows permutes whole blocks: the exact mean cannot change
    perm = torch.randperm(2048, generator=torch.Generator().manual_seed(0)).to(d)
    c = dg.nf4_quantize(W[perm].contiguous())
    torch.cuda.synchronize()
    assert u32(c.absmax_mean)[0] == u32(a.absmax_mean)[0]


def _blocks_with_absmax(values, seed):
    """A fp32 weight whose 64-blocks have exactly the given absmax values."""
    rng = np.random.default_rng(seed)
    a = np.asarray(values, np.float32)
    w = (rng.uniform(-1, 1, (a.size, 64)) * a[:, None]).astype(np.float32)
    w[:, 5] = a                       # the block maximum, attained exactly
    w = np.minimum(np.maximum(w, -a[:, None]), a[:, None])
    return torch.from_numpy(w)


@pytest.mark.parametrize("case", ["subnormal", "huge", "wide", "tie_even", "tie_odd", "single"])
def test_exact_mean_edge_cases(case):
    """The device's exact mean against the oracle where rounding is delicate."""
    rng = np.random.default_rng(7)
    one = np.float32(1.0)
    up = np.nextafter(one, np.float32(2))
    if case == "subnormal":
        vals = (np.abs(rng.standard_normal(777)) * 1e-41).astype(np.float32) + np.float32(1e-45)
    elif case == "huge":
        vals = np.float32(3.0e38) - (np.abs(rng.standard_normal(300)) * 1e36).astype(np.float32)
    elif case == "wide":
        vals = np.abs(rng.standard_normal(2000) * 10.0 ** rng.integers(-37, 37, 2000)).astype(np.float32)
    elif case == "tie_even":
        vals = np.array([one, up], np.float32)           # mean 1 + 2^-24: a tie, rounds to 1.0
    elif case == "tie_odd":
        vals = np.array([up, np.nextafter(up, np.float32(2))], np.float32)  # tie, rounds up to even
    else:
        vals = np.array([np.float32(0.123)], np.float32)
    _check_roundtrip(_blocks_with_absmax(vals, 3), True, f"mean {case}")


@pytest.mark.parametrize("dq", [True, False])
def test_decode_weight_full(dq):
    _check_roundtrip(synth.decode_weight(0), dq, f"decode dq={dq}")


def test_prefill_weight_full():
    note("prefill weight 11008x4096: oracle over every element")
    _check_roundtrip(synth.prefill_weight(), True, "prefill")


def test_large_outlier_weight(large_oracle):
    """28672x8192 fp32 Student-t(4): every code, the absmax state and every W^ element."""
    dg = lib()
    d = dev()
    W, qo = large_oracle
    note("large weight: GPU quantize and dequantize")
    qg = dg.nf4_quantize(W.to(d), double_quant=True)
    wh = dg.nf4_dequantize(qg, torch.bfloat16)
    torch.cuda.synchronize()
    assert_quant_equal(qg, qo, "large")
    note("large weight: packed codes and int8 state bit-exact; oracle W^")
    want = O.dequantize(qo)
    bad = np.count_nonzero(bf16_bits(wh).ravel() != want)
    assert bad == 0, f"large: {bad} bf16 W^ differ"


def _oracle_roundtrip(W):
    """The oracle's quantization and bf16 W^ of one matrix (run on a worker thread)."""
    qo = oracle_quantize(W, True)
    return qo, O.dequantize(qo)


@pytest.mark.parametrize("layers", [range(0, 8), range(8, 16), range(16, 24), range(24, 32)])
def test_bulk_decoder_layers(layers):
    """Bulk: every linear of a 32-layer decoder, every element.

    Each matrix is quantized and dequantized on the GPU and compared bit for bit
    with the oracle: packed codes, int8 absmax, scales, mean and bf16 W^.  The
    oracle runs on a thread pool, one matrix per task, while the GPU works
    through the same matrices.
    """
    dg = lib()
    d = dev()
    for l in layers:
        keys = [(l, j) for j in range(7)]
        mats = synth.bulk_weights_parallel(keys)
        with cf.ThreadPoolExecutor(max_workers=_workers()) as ex:
            fut = {k: ex.submit(_oracle_roundtrip, mats[k]) for k in keys}
            for (_, j) in keys:
                W = mats[(l, j)]
                where = f"bulk layer {l} {synth.BULK_NAMES[j]}"
                qg = dg.nf4_quantize(W.to(d), double_quant=True)
                wh = dg.nf4_dequantize(qg, torch.bfloat16)
                torch.cuda.synchronize()
                qo, want = fut[(l, j)].result()
                assert_quant_equal(qg, qo, where)
                bad = np.count_nonzero(bf16_bits(wh).ravel() != want)
                assert bad == 0, f"{where}: {bad} bf16 W^ differ"
                del qg, wh
        note(f"bulk layer {l}: 7 matrices bit-exact on every element")


def _workers():
    return max(1, min(16, len(os.sched_getaffinity(0))))
