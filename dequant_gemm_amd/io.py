"""Saving and loading NF4-quantized weights (the QuantState's persistent form).

"bitsandbytes" page, QuantState paragraph: a quantized tensor travels with its
quantization state -- the packed data, the absmax values and the shape and
dtype needed to restore it.  Here that is a :class:`QTensor`: packed codes,
int8 absmax with fp32 scales and the fp32 mean (double quantization) or fp32
absmax, plus rows, cols and the block size.

Files are safetensors (no code is executed on load).  Each weight ``name``
stores ``name.packed`` (uint8), ``name.absmax_q`` (int8), ``name.absmax_scale``
(fp32) and ``name.absmax_mean`` (fp32 [1]), or ``name.absmax`` (fp32) without
double quantization; the file metadata records, per weight, rows, cols, block
size, double quantization and the 4-bit data type (NF4 or FP4; the same
paragraph has the data type travel with the state), and once the bit
patterns of both 16-level tables the codes index.  Loading checks every
buffer size against the shape and refuses a file written with another level
table.  The round trip is bit-exact.
"""
from __future__ import annotations

import json
from typing import Dict

import torch

from ._lib import BLOCKSIZES, QUANT_TYPES, QTensor, nf4_levels, nf4_sizes

FORMAT = "nf4-qtensor"
VERSION = "1"
_FIELDS = ("packed", "absmax", "absmax_q", "absmax_scale", "absmax_mean")
_DTYPES = {"packed": torch.uint8, "absmax": torch.float32, "absmax_q": torch.int8,
           "absmax_scale": torch.float32, "absmax_mean": torch.float32}


def _codebook_hex(quant_type: str = "nf4") -> str:
    return "".join(f"{b & 0xFFFFFFFF:08x}" for b in nf4_levels(quant_type).view(torch.int32).tolist())


def _expected_sizes(rows: int, cols: int, blocksize: int, dq: bool) -> Dict[str, int]:
    s = nf4_sizes(rows, cols, blocksize, dq)
    if dq:
        return {"packed": s["packed_bytes"], "absmax_q": s["nblocks"], "absmax_scale": s["ngroups"],
                "absmax_mean": 1}
    return {"packed": s["packed_bytes"], "absmax": s["nblocks"]}


def qtensor_state(name: str, q: QTensor) -> tuple[Dict[str, torch.Tensor], Dict[str, dict]]:
    """The tensors (on the host) and metadata entries that represent ``q``."""
    tensors = {}
    for f in _FIELDS:
        t = getattr(q, f)
        if t is not None:
            tensors[f"{name}.{f}"] = t.detach().to("cpu").contiguous()
    meta = {name: {"rows": q.rows, "cols": q.cols, "blocksize": q.blocksize,
                   "double_quant": bool(q.double_quant), "quant_type": q.quant_type}}
    return tensors, meta


def save_qtensors(path: str, weights: Dict[str, QTensor]) -> None:
    """Writes several quantized weights, keyed by name, to one safetensors file."""
    from safetensors.torch import save_file
    tensors: Dict[str, torch.Tensor] = {}
    entries: Dict[str, dict] = {}
    for name, q in weights.items():
        if "." in name and any(name.endswith("." + f) for f in _FIELDS):
            raise ValueError(f"weight name {name!r} ends like a buffer name")
        t, m = qtensor_state(name, q)
        tensors.update(t)
        entries.update(m)
    meta = {"format": FORMAT, "version": VERSION, "levels": _codebook_hex("nf4"),
            "levels_fp4": _codebook_hex("fp4"), "weights": json.dumps(entries)}
    save_file(tensors, path, metadata=meta)


def save_qtensor(path: str, q: QTensor, name: str = "weight") -> None:
    save_qtensors(path, {name: q})


def load_qtensors(path: str, device="cpu") -> Dict[str, QTensor]:
    """Reads every quantized weight of a file written by :func:`save_qtensors`."""
    from safetensors import safe_open
    out: Dict[str, QTensor] = {}
    with safe_open(path, framework="pt", device="cpu") as f:
        meta = f.metadata() or {}
        if meta.get("format") != FORMAT or meta.get("version") != VERSION:
            raise ValueError(f"{path}: not an {FORMAT} v{VERSION} file")
        if meta.get("levels") != _codebook_hex("nf4"):
            raise ValueError(f"{path}: written with a different NF4 level table")
        entries = json.loads(meta["weights"])
        keys = set(f.keys())
        for name, e in entries.items():
            rows, cols, bs, dq = int(e["rows"]), int(e["cols"]), int(e["blocksize"]), bool(e["double_quant"])
            if bs not in BLOCKSIZES:
                raise ValueError(f"{path}: {name} has block size {bs}; supported: {BLOCKSIZES}")
            qt = e.get("quant_type", "nf4")
            if qt not in QUANT_TYPES:
                raise ValueError(f"{path}: {name} has quant_type {qt!r}; supported: {tuple(QUANT_TYPES)}")
            if qt == "fp4" and meta.get("levels_fp4") != _codebook_hex("fp4"):
                raise ValueError(f"{path}: written with a different FP4 level table")
            want = _expected_sizes(rows, cols, bs, dq)
            bufs = {}
            for fld, n in want.items():
                key = f"{name}.{fld}"
                if key not in keys:
                    raise ValueError(f"{path}: {key} is missing")
                t = f.get_tensor(key)
                if t.dtype != _DTYPES[fld] or t.dim() != 1 or t.numel() != n:
                    raise ValueError(f"{path}: {key} is {t.dtype} {tuple(t.shape)}, expected {_DTYPES[fld]} ({n},)")
                bufs[fld] = t.to(device)
            out[name] = QTensor(rows, cols, dq, blocksize=bs, quant_type=qt, **bufs)
    return out


def load_qtensor(path: str, name: str = "weight", device="cpu") -> QTensor:
    ws = load_qtensors(path, device)
    if name not in ws:
        raise KeyError(f"{path}: no weight named {name!r}")
    return ws[name]
