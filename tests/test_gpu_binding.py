"""The binding refuses buffers the kernels would overrun, before anything launches.

The C ABI takes raw device pointers and cannot see buffer sizes.  The Python
binding therefore checks every output buffer, and every buffer of a quantized
weight, against the sizes, dtypes and device that the call implies, and raises
ValueError.  Each refused case below would otherwise read or write past the end
of a buffer; each check also confirms that a refused call left its output
untouched.
"""
import dataclasses

import pytest
import torch

import synth
from tests._gpu import dev, lib

pytestmark = pytest.mark.gpu
BF = torch.bfloat16


def _setup(double_quant=True):
    dg, d = lib(), dev()
    W = synth.normal((64, 256), 0.02, 600).to(d)
    q = dg.nf4_quantize(W, double_quant=double_quant)
    torch.cuda.synchronize()
    return dg, d, W, q


def _refused(fn, out=None):
    before = None if out is None else out.clone()
    with pytest.raises(ValueError):
        fn()
    if out is not None:
        torch.cuda.synchronize()
        assert torch.equal(out, before)


def test_short_or_strided_outputs_are_refused():
    dg, d, W, q = _setup()
    X = torch.ones((8, 256), dtype=BF, device=d)
    dY = torch.ones((8, 64), dtype=BF, device=d)
    U, B = torch.ones((8, 16), dtype=BF, device=d), torch.ones((64, 16), dtype=BF, device=d)
    V, At = torch.ones((8, 16), dtype=BF, device=d), torch.ones((256, 16), dtype=BF, device=d)
    o = torch.full((64 * 256 - 1,), 7.0, dtype=BF, device=d)
    _refused(lambda: dg.nf4_dequantize(q, out=o), o)
    o = torch.full((8, 63), 7.0, device=d)
    _refused(lambda: dg.nf4_matmul_fwd(X, q, out=o), o)
    _refused(lambda: dg.nf4_matmul_fwd_lora(X, q, U, B, out=o), o)
    o = torch.full((7, 256), 7.0, device=d)
    _refused(lambda: dg.nf4_matmul_bwd_dx(dY, q, out=o), o)
    _refused(lambda: dg.nf4_matmul_bwd_dx_lora(dY, q, V, At, out=o), o)
    o = torch.full((64, 8), 7.0, device=d)
    _refused(lambda: dg.nf4_matmul_fwd(X, q, out=o.t()), o)          # right size, not contiguous
    # the same calls with correct buffers go through
    Y = dg.nf4_matmul_fwd(X, q, out=torch.empty((8, 64), device=d))
    dX = dg.nf4_matmul_bwd_dx(dY, q, out=torch.empty((8, 256), device=d))
    torch.cuda.synchronize()
    assert Y.shape == (8, 64) and dX.shape == (8, 256)


@pytest.mark.parametrize("double_quant", [True, False])
def test_short_or_mistyped_weight_buffers_are_refused(double_quant):
    dg, d, W, q = _setup(double_quant)
    X = torch.ones((8, 256), dtype=BF, device=d)
    names = ("packed", "absmax_q", "absmax_scale", "absmax_mean") if double_quant else ("packed", "absmax")
    for name in names:
        short = dataclasses.replace(q, **{name: getattr(q, name)[:-1]})
        missing = dataclasses.replace(q, **{name: None})
        for bad in (short, missing):
            o = torch.full((64, 256), 7.0, dtype=BF, device=d)
            _refused(lambda: dg.nf4_dequantize(bad, out=o), o)
            _refused(lambda: dg.nf4_matmul_fwd(X, bad))
            keep = getattr(q, name).clone()
            _refused(lambda: dg.nf4_quantize(W, out=bad, double_quant=double_quant))
            torch.cuda.synchronize()
            assert torch.equal(getattr(q, name), keep)
    wrong = "absmax_scale" if double_quant else "absmax"
    retyped = dataclasses.replace(q, **{wrong: getattr(q, wrong).view(torch.int32)})
    _refused(lambda: dg.nf4_matmul_fwd(X, retyped))


def test_status_word_and_devices():
    dg, d, W, q = _setup()
    _refused(lambda: dg.nf4_quantize(W, status=torch.zeros(0, dtype=torch.int32, device=d)))
    _refused(lambda: dg.nf4_quantize(W, status=torch.zeros(1, dtype=torch.int32)))          # host memory
    X = torch.ones((8, 256), dtype=BF, device=d)
    _refused(lambda: dg.nf4_matmul_fwd(X.cpu(), q))
    U, B = torch.ones((8, 16), dtype=BF), torch.ones((64, 16), dtype=BF, device=d)
    _refused(lambda: dg.nf4_matmul_fwd_lora(X, q, U, B))
