"""The allocation-free quantize entry point against nf4_quantize, through the C ABI.

nf4_quantize_noalloc must produce exactly what nf4_quantize (with a caller
workspace) produces: packed codes, int8 absmax, scales and mean (or the fp32
absmax without double quantization), bit for bit.  Its scratch is one fixed
buffer per GPU that keeps the previous call's contents, so the calls come in
sequences whose later inputs are smaller than the earlier ones.
"""
import pytest
import torch

import synth
from tests._gpu import dev, lib, note

pytestmark = pytest.mark.gpu

_FIELDS = ("packed", "absmax", "absmax_q", "absmax_scale", "absmax_mean")


def _poisoned(dg, rows, cols, dq, bs, qt, d):
    """An output descriptor whose buffers hold a fill pattern, so a byte left unwritten shows."""
    q = dg.empty_qtensor(rows, cols, dq, d, bs, qt)
    for f in _FIELDS:
        t = getattr(q, f)
        if t is not None:
            t.view(torch.uint8).fill_(0xA5)
    return q


def _same_as_workspace_call(W, bs=64, dq=True, qt="nf4"):
    dg = lib()
    d = dev()
    rows, cols = W.shape
    note(f"noalloc: {rows}x{cols} {W.dtype} bs={bs} dq={dq} {qt}")
    ref = dg.empty_qtensor(rows, cols, dq, d, bs, qt)
    out = _poisoned(dg, rows, cols, dq, bs, qt, d)
    st_ref = torch.zeros(4, dtype=torch.int32, device=d)
    st = torch.zeros(4, dtype=torch.int32, device=d)
    dg.nf4_quantize(W, blocksize=bs, double_quant=dq, quant_type=qt, out=ref, status=st_ref)
    dg.nf4_quantize_noalloc(W, out, status=st)
    torch.cuda.synchronize()
    for f in _FIELDS:
        a, b = getattr(ref, f), getattr(out, f)
        assert (a is None) == (b is None), f
        if a is not None:
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), f"{rows}x{cols} bs={bs} {qt}: {f} differs"
    assert torch.equal(st, st_ref)


@pytest.mark.parametrize("qt", ["nf4", "fp4"])
def test_two_calls_second_smaller(qt):
    """A prefill-sized weight, then a ragged one with a partial last block and group."""
    d = dev()
    _same_as_workspace_call(synth.prefill_weight().to(d), qt=qt)
    _same_as_workspace_call(synth.normal((300, 777), 0.02, 5, torch.float32).to(d), qt=qt)


def test_block_sizes_and_no_double_quant():
    d = dev()
    W = synth.normal((2048, 4096), 0.02, 6).to(d)
    for bs in (256, 128, 64, 32):
        _same_as_workspace_call(W, bs=bs)
    _same_as_workspace_call(W, dq=False)
    _same_as_workspace_call(W[:37].contiguous(), bs=32)


def test_largest_tensor_the_scratch_holds():
    """NF4_NOALLOC_MAX_BLOCKS blocks exactly (2^28 bf16 weights at block size 64), then a small one."""
    dg = lib()
    d = dev()
    cols = 4096
    rows = dg.NOALLOC_MAX_BLOCKS * 64 // cols
    g = torch.Generator(device=d)
    g.manual_seed(77)
    W = (torch.randn((rows, cols), generator=g, device=d) * 0.02).to(torch.bfloat16)
    _same_as_workspace_call(W)
    del W
    torch.cuda.empty_cache()
    _same_as_workspace_call(synth.normal((64, 320), 0.02, 8).to(d))
