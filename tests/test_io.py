"""Save/load of quantized weights ("bitsandbytes" page, QuantState paragraph).

CPU only: the state written is the oracle's quantization of a seeded weight,
held in host tensors; the file is read back and every buffer must be
bit-identical.  Malformed files must be refused.
"""
import json

import numpy as np
import pytest
import torch

import oracle as O
import synth
from dequant_gemm_amd import QTensor
from dequant_gemm_amd.io import load_qtensor, load_qtensors, save_qtensor, save_qtensors


def _oracle_qtensor(rows, cols, dq, seed, quant_type="nf4"):
    W = synth.normal((rows, cols), 0.02, seed, torch.float32)
    qo = O.quantize(W.numpy(), double_quant_on=dq, quant_type=quant_type)
    q = QTensor(rows, cols, dq, torch.from_numpy(qo["packed"].copy()), quant_type=quant_type)
    if dq:
        q.absmax_q = torch.from_numpy(qo["absmax_q"].astype(np.int8))
        q.absmax_scale = torch.from_numpy(qo["scale"].astype(np.float32))
        q.absmax_mean = torch.tensor([qo["mean"]], dtype=torch.float32)
    else:
        q.absmax = torch.from_numpy(qo["absmax"].astype(np.float32))
    return q


def _same(a: QTensor, b: QTensor):
    assert (a.rows, a.cols, a.double_quant, a.blocksize, a.quant_type) == \
        (b.rows, b.cols, b.double_quant, b.blocksize, b.quant_type)
    for f in ("packed", "absmax", "absmax_q", "absmax_scale", "absmax_mean"):
        x, y = getattr(a, f), getattr(b, f)
        assert (x is None) == (y is None), f
        if x is not None:
            assert x.dtype == y.dtype and torch.equal(x.view(torch.uint8), y.view(torch.uint8)), f


@pytest.mark.parametrize("dq", [True, False])
def test_round_trip_bit_exact(tmp_path, dq):
    q = _oracle_qtensor(256, 256, dq, 0)
    p = str(tmp_path / "w.safetensors")
    save_qtensor(p, q)
    _same(q, load_qtensor(p))


def test_several_weights_and_ragged(tmp_path):
    ws = {"layers.0.q_proj": _oracle_qtensor(64, 128, True, 1),
          "layers.0.down": _oracle_qtensor(3, 37, False, 2),      # partial block, odd numel
          "lm": _oracle_qtensor(300, 777, True, 3)}               # partial double-quant group
    p = str(tmp_path / "m.safetensors")
    save_qtensors(p, ws)
    back = load_qtensors(p)
    assert set(back) == set(ws)
    for k in ws:
        _same(ws[k], back[k])


def test_fp4_weights_keep_their_data_type(tmp_path):
    ws = {"a": _oracle_qtensor(64, 128, True, 5, "fp4"), "b": _oracle_qtensor(33, 65, False, 6, "fp4"),
          "c": _oracle_qtensor(64, 64, True, 7, "nf4")}
    p = str(tmp_path / "mixed.safetensors")
    save_qtensors(p, ws)
    back = load_qtensors(p)
    for k in ws:
        _same(ws[k], back[k])
    assert [back[k].quant_type for k in ("a", "b", "c")] == ["fp4", "fp4", "nf4"]
    bad = str(tmp_path / "bad.safetensors")

    def other_fp4_levels(m):
        m["levels_fp4"] = "0" * 128
        return m
    _rewrite(p, bad, meta_fn=other_fp4_levels)
    with pytest.raises(ValueError, match="FP4 level table"):
        load_qtensors(bad)

    def unknown_type(m):
        e = json.loads(m["weights"])
        e["a"]["quant_type"] = "int4"
        m["weights"] = json.dumps(e)
        return m
    _rewrite(p, bad, meta_fn=unknown_type)
    with pytest.raises(ValueError, match="quant_type"):
        load_qtensors(bad)


def test_entries_without_a_data_type_load_as_nf4(tmp_path):
    p = str(tmp_path / "old.safetensors")
    save_qtensor(p, _oracle_qtensor(64, 64, True, 8))
    bad = str(tmp_path / "noqt.safetensors")

    def drop(m):
        e = json.loads(m["weights"])
        del e["weight"]["quant_type"]
        m["weights"] = json.dumps(e)
        return m
    _rewrite(p, bad, meta_fn=drop)
    assert load_qtensor(bad).quant_type == "nf4"


def _rewrite(src, dst, tensors_fn=None, meta_fn=None):
    from safetensors import safe_open
    from safetensors.torch import save_file
    with safe_open(src, framework="pt") as f:
        meta = dict(f.metadata())
        tensors = {k: f.get_tensor(k) for k in f.keys()}
    if tensors_fn:
        tensors = tensors_fn(tensors)
    if meta_fn:
        meta = meta_fn(meta)
    save_file(tensors, dst, metadata=meta)


def test_refuses_malformed(tmp_path):
    q = _oracle_qtensor(64, 64, True, 4)
    p = str(tmp_path / "ok.safetensors")
    save_qtensor(p, q)
    bad = str(tmp_path / "bad.safetensors")

    def other_levels(m):
        m["levels"] = "0" * 128
        return m
    _rewrite(p, bad, meta_fn=other_levels)
    with pytest.raises(ValueError, match="level table"):
        load_qtensor(bad)

    def short_packed(t):
        t["weight.packed"] = t["weight.packed"][:-1].clone()
        return t
    _rewrite(p, bad, tensors_fn=short_packed)
    with pytest.raises(ValueError, match="packed"):
        load_qtensor(bad)

    def no_scale(t):
        del t["weight.absmax_scale"]
        return t
    _rewrite(p, bad, tensors_fn=no_scale)
    with pytest.raises(ValueError, match="missing"):
        load_qtensor(bad)

    def wrong_dtype(t):
        t["weight.absmax_q"] = t["weight.absmax_q"].to(torch.int16)
        return t
    _rewrite(p, bad, tensors_fn=wrong_dtype)
    with pytest.raises(ValueError, match="absmax_q"):
        load_qtensor(bad)

    def other_blocksize(m):
        e = json.loads(m["weights"])
        e["weight"]["blocksize"] = 48
        m["weights"] = json.dumps(e)
        return m
    _rewrite(p, bad, meta_fn=other_blocksize)
    with pytest.raises(ValueError, match="block size"):
        load_qtensor(bad)

    def not_ours(m):
        m["format"] = "something-else"
        return m
    _rewrite(p, bad, meta_fn=not_ours)
    with pytest.raises(ValueError, match="not an"):
        load_qtensor(bad)

    with pytest.raises(KeyError):
        load_qtensor(p, name="nope")
