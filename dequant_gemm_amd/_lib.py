"""ctypes binding of libnf4.so (the C ABI in include/nf4.h).

Argument marshalling only: every step of quantization, dequantization and the
GEMMs runs in the library's HIP kernels.  torch supplies device memory
(``data_ptr()``) and the current HIP stream; nothing else.  There is no CPU
fallback: if the library is missing or a call fails, a ``RuntimeError`` is
raised.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libnf4.so")

NF4_OK = 0
NF4_F32 = 0
NF4_BF16 = 1
BLOCKSIZE = 64
BLOCKSIZES = (32, 64, 128, 256)
DQ_GROUP = 256
QUANT_TYPES = {"nf4": 0, "fp4": 1}     # nf4_quant_type: the level table

STATUS_NAMES = {
    0: "NF4_OK", 1: "NF4_ERR_NULL", 2: "NF4_ERR_SHAPE", 3: "NF4_ERR_BLOCKSIZE", 4: "NF4_ERR_DTYPE",
    5: "NF4_ERR_ALIGN", 6: "NF4_ERR_WORKSPACE", 7: "NF4_ERR_UNSUPPORTED", 8: "NF4_ERR_HIP",
    9: "NF4_ERR_QUANT_TYPE", 10: "NF4_ERR_SCRATCH",
}

EXPORTS = ("nf4_status_string", "nf4_codebook", "nf4_levels", "nf4_thresholds", "nf4_sizes", "nf4_quantize",
           "nf4_quantize_noalloc", "nf4_dequantize", "nf4_matmul_fwd", "nf4_matmul_bwd_dx", "nf4_matmul_fwd_lora",
           "nf4_matmul_bwd_dx_lora", "nf4_adapter_matmul")
LORA_RANK_STEP = 16
LORA_MAX_RANK = 1024
NOALLOC_MAX_BLOCKS = 1 << 22     # NF4_NOALLOC_MAX_BLOCKS: blocks nf4_quantize_noalloc's scratch holds


class QTensorStruct(ctypes.Structure):
    """Mirror of ``nf4_qtensor``."""
    _fields_ = [
        ("rows", ctypes.c_int64), ("cols", ctypes.c_int64),
        ("blocksize", ctypes.c_int32), ("double_quant", ctypes.c_int32),
        ("packed", ctypes.c_void_p), ("absmax", ctypes.c_void_p), ("absmax_q", ctypes.c_void_p),
        ("absmax_scale", ctypes.c_void_p), ("absmax_mean", ctypes.c_void_p),
        ("quant_type", ctypes.c_int32),
    ]


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libnf4.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m dequant_gemm_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, i64, i32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t
        L.nf4_status_string.argtypes = [i32]
        L.nf4_status_string.restype = ctypes.c_char_p
        L.nf4_codebook.argtypes = [ctypes.POINTER(ctypes.c_float)]
        L.nf4_levels.argtypes = [i32, ctypes.POINTER(ctypes.c_float)]
        L.nf4_thresholds.argtypes = [ctypes.POINTER(ctypes.c_float)]
        L.nf4_sizes.argtypes = [i64, i64, i32, i32, ctypes.POINTER(i64), ctypes.POINTER(i64),
                                ctypes.POINTER(i64), ctypes.POINTER(sz)]
        L.nf4_quantize.argtypes = [vp, i32, i64, i64, i32, i32, ctypes.POINTER(QTensorStruct), vp, sz, vp, vp]
        L.nf4_quantize_noalloc.argtypes = [vp, i32, i64, i64, i32, i32, ctypes.POINTER(QTensorStruct), vp, vp]
        L.nf4_dequantize.argtypes = [ctypes.POINTER(QTensorStruct), vp, i32, vp]
        L.nf4_matmul_fwd.argtypes = [vp, i64, ctypes.POINTER(QTensorStruct), vp, i32, vp]
        L.nf4_matmul_bwd_dx.argtypes = [vp, i64, ctypes.POINTER(QTensorStruct), vp, i32, vp]
        L.nf4_matmul_fwd_lora.argtypes = [vp, i64, ctypes.POINTER(QTensorStruct), vp, vp, i64, vp, i32, vp]
        L.nf4_matmul_bwd_dx_lora.argtypes = [vp, i64, ctypes.POINTER(QTensorStruct), vp, vp, i64, vp, i32, vp]
        L.nf4_adapter_matmul.argtypes = [i32, i32, i64, i64, i64, ctypes.c_float, vp, i64, vp, i64, vp, i32, i64, vp]
        for name in EXPORTS[1:]:
            getattr(L, name).restype = i32
        _lib = L
    return _lib


class NF4Error(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = lib().nf4_status_string(status).decode()
        super().__init__(f"{where}: {STATUS_NAMES.get(status, status)} ({msg})")


def _check(status: int, where: str):
    if status != NF4_OK:
        raise NF4Error(status, where)


def _dtype_enum(dt: torch.dtype) -> int:
    if dt == torch.float32:
        return NF4_F32
    if dt == torch.bfloat16:
        return NF4_BF16
    raise TypeError(f"unsupported dtype {dt}; use torch.float32 or torch.bfloat16")


def _stream(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _require_device(t: torch.Tensor, name: str):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device (HIP) tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _require_out(out: torch.Tensor, numel: int, device: torch.device, name: str = "out"):
    """An output buffer the kernels will fill: contiguous, on ``device``, exactly ``numel`` elements.

    The C ABI takes raw pointers and cannot see buffer sizes; this is where a
    too-small buffer is caught before anything is written.
    """
    _require_device(out, name)
    if out.device != device:
        raise ValueError(f"{name} is on {out.device}, the operands on {device}")
    if out.numel() != numel:
        raise ValueError(f"{name} has {out.numel()} elements, the result {numel}")


def _quant_type_enum(quant_type: str) -> int:
    if quant_type not in QUANT_TYPES:
        raise ValueError(f"quant_type must be one of {tuple(QUANT_TYPES)} (got {quant_type!r})")
    return QUANT_TYPES[quant_type]


@dataclass
class QTensor:
    """A 4-bit quantized weight [rows, cols] (the QuantState analogue).

    Device buffers: ``packed`` (uint8, ceil(numel/2)); without double
    quantization ``absmax`` (fp32 per block); with it ``absmax_q`` (int8 per
    block), ``absmax_scale`` (fp32 per 256 blocks) and ``absmax_mean`` (fp32 [1]).
    ``quant_type`` names the level table: "nf4" (default) or "fp4".
    """
    rows: int
    cols: int
    double_quant: bool
    packed: torch.Tensor
    absmax: Optional[torch.Tensor] = None
    absmax_q: Optional[torch.Tensor] = None
    absmax_scale: Optional[torch.Tensor] = None
    absmax_mean: Optional[torch.Tensor] = None
    blocksize: int = BLOCKSIZE
    quant_type: str = "nf4"

    @property
    def shape(self):
        return (self.rows, self.cols)

    @property
    def device(self):
        if self.packed is None:
            raise ValueError("QTensor.packed is missing")
        return self.packed.device

    def check(self):
        """Buffer dtypes, devices and sizes against rows, cols, blocksize and double_quant."""
        numel = self.rows * self.cols
        nb = -(-numel // self.blocksize) if self.blocksize > 0 else 0
        want = [("packed", self.packed, torch.uint8, -(-numel // 2))]
        if self.double_quant:
            want += [("absmax_q", self.absmax_q, torch.int8, nb),
                     ("absmax_scale", self.absmax_scale, torch.float32, -(-nb // DQ_GROUP)),
                     ("absmax_mean", self.absmax_mean, torch.float32, 1)]
        else:
            want.append(("absmax", self.absmax, torch.float32, nb))
        for name, t, dt, n in want:
            if t is None:
                raise ValueError(f"QTensor.{name} is missing")
            _require_device(t, f"QTensor.{name}")
            if t.device != self.packed.device:
                raise ValueError(f"QTensor.{name} is on {t.device}, packed on {self.packed.device}")
            if t.dtype != dt or t.numel() < n:
                raise ValueError(f"QTensor.{name} must be {dt} with at least {n} elements "
                                 f"(got {t.dtype}, {t.numel()})")

    def struct(self) -> QTensorStruct:
        self.check()
        return QTensorStruct(self.rows, self.cols, self.blocksize, int(self.double_quant),
                             _ptr(self.packed), _ptr(self.absmax), _ptr(self.absmax_q),
                             _ptr(self.absmax_scale), _ptr(self.absmax_mean),
                             _quant_type_enum(self.quant_type))

    def nbytes(self) -> int:
        return sum(t.numel() * t.element_size() for t in
                   (self.packed, self.absmax, self.absmax_q, self.absmax_scale, self.absmax_mean) if t is not None)


# ------------------------------------------------------------------ the C ABI, by name

def nf4_codebook() -> torch.Tensor:
    out = (ctypes.c_float * 16)()
    _check(lib().nf4_codebook(out), "nf4_codebook")
    return torch.tensor(list(out), dtype=torch.float32)


def nf4_levels(quant_type: str = "nf4") -> torch.Tensor:
    """The 16 levels of ``quant_type`` indexed by code (NF4 ascending; FP4 by E2M1 bit pattern)."""
    out = (ctypes.c_float * 16)()
    _check(lib().nf4_levels(_quant_type_enum(quant_type), out), "nf4_levels")
    return torch.tensor(list(out), dtype=torch.float32)


def nf4_thresholds() -> torch.Tensor:
    out = (ctypes.c_float * 15)()
    _check(lib().nf4_thresholds(out), "nf4_thresholds")
    return torch.tensor(list(out), dtype=torch.float32)


def nf4_sizes(rows: int, cols: int, blocksize: int = BLOCKSIZE, double_quant: bool = True) -> dict:
    pb, nb, ng = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
    ws = ctypes.c_size_t()
    _check(lib().nf4_sizes(rows, cols, blocksize, int(double_quant), ctypes.byref(pb), ctypes.byref(nb),
                           ctypes.byref(ng), ctypes.byref(ws)), "nf4_sizes")
    return {"packed_bytes": pb.value, "nblocks": nb.value, "ngroups": ng.value, "workspace_bytes": ws.value}


def empty_qtensor(rows: int, cols: int, double_quant: bool = True, device="cuda",
                  blocksize: int = BLOCKSIZE, quant_type: str = "nf4") -> QTensor:
    _quant_type_enum(quant_type)
    s = nf4_sizes(rows, cols, blocksize, double_quant)
    dev = torch.device(device)
    q = QTensor(rows, cols, double_quant, torch.empty(s["packed_bytes"], dtype=torch.uint8, device=dev),
                blocksize=blocksize, quant_type=quant_type)
    if double_quant:
        q.absmax_q = torch.empty(s["nblocks"], dtype=torch.int8, device=dev)
        q.absmax_scale = torch.empty(s["ngroups"], dtype=torch.float32, device=dev)
        q.absmax_mean = torch.empty(1, dtype=torch.float32, device=dev)
    else:
        q.absmax = torch.empty(s["nblocks"], dtype=torch.float32, device=dev)
    return q


def nf4_quantize(W: torch.Tensor, blocksize: int = BLOCKSIZE, double_quant: bool = True,
                 out: Optional[QTensor] = None, workspace: Optional[torch.Tensor] = None,
                 status: Optional[torch.Tensor] = None, quant_type: Optional[str] = None) -> QTensor:
    """4-bit quantize a 2-D bf16/fp32 device tensor (row-major flattening).

    ``quant_type`` is "nf4" (default) or "fp4"; with ``out`` it defaults to
    ``out.quant_type`` and must agree with it.
    """
    _require_device(W, "W")
    if W.dim() != 2:
        raise ValueError("W must be 2-D [rows, cols]")
    rows, cols = W.shape
    if out is not None:
        if quant_type is not None and quant_type != out.quant_type:
            raise ValueError(f"quant_type {quant_type!r} does not match out.quant_type {out.quant_type!r}")
        q = out
    else:
        q = empty_qtensor(rows, cols, double_quant, W.device, blocksize, quant_type or "nf4")
    s = nf4_sizes(rows, cols, blocksize, double_quant)
    if workspace is None and s["workspace_bytes"]:
        workspace = torch.empty(s["workspace_bytes"], dtype=torch.uint8, device=W.device)
    if q.device != W.device:
        raise ValueError(f"out is on {q.device}, W on {W.device}")
    for t, nm in ((workspace, "workspace"), (status, "status")):
        if t is not None:
            _require_device(t, nm)
            if t.device != W.device:
                raise ValueError(f"{nm} is on {t.device}, W on {W.device}")
    if status is not None and status.numel() * status.element_size() < 4:
        raise ValueError("status must hold at least one uint32")
    st = q.struct()
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().nf4_quantize(W.data_ptr(), _dtype_enum(W.dtype), rows, cols, blocksize, int(double_quant),
                              ctypes.byref(st), _ptr(workspace), ws_bytes, _ptr(status), _stream(W.device)),
           "nf4_quantize")
    return q


def nf4_quantize_noalloc(W: torch.Tensor, out: QTensor, status: Optional[torch.Tensor] = None) -> QTensor:
    """``nf4_quantize`` into the caller's ``out`` without a workspace: the library's fixed
    per-GPU scratch serves instead, so the C call allocates nothing (block size, double
    quantization and quant_type come from ``out``)."""
    _require_device(W, "W")
    if W.dim() != 2:
        raise ValueError("W must be 2-D [rows, cols]")
    rows, cols = W.shape
    if out.device != W.device:
        raise ValueError(f"out is on {out.device}, W on {W.device}")
    if status is not None:
        _require_device(status, "status")
        if status.device != W.device:
            raise ValueError(f"status is on {status.device}, W on {W.device}")
        if status.numel() * status.element_size() < 4:
            raise ValueError("status must hold at least one uint32")
    st = out.struct()
    _check(lib().nf4_quantize_noalloc(W.data_ptr(), _dtype_enum(W.dtype), rows, cols, out.blocksize,
                                      int(out.double_quant), ctypes.byref(st), _ptr(status), _stream(W.device)),
           "nf4_quantize_noalloc")
    return out


def nf4_dequantize(q: QTensor, dtype: torch.dtype = torch.bfloat16, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    if out is None:
        out = torch.empty((q.rows, q.cols), dtype=dtype, device=q.device)
    _require_out(out, q.rows * q.cols, q.device)
    st = q.struct()
    _check(lib().nf4_dequantize(ctypes.byref(st), out.data_ptr(), _dtype_enum(out.dtype), _stream(q.device)),
           "nf4_dequantize")
    return out


def nf4_matmul_fwd(X: torch.Tensor, q: QTensor, out_dtype: torch.dtype = torch.float32,
                   out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Y = X W^T with W^ dequantized on chip.  X: bf16 [M, K] (K = q.cols)."""
    _require_device(X, "X")
    if X.dtype != torch.bfloat16 or X.dim() != 2 or X.shape[1] != q.cols:
        raise ValueError("X must be bf16 [M, q.cols]")
    M = X.shape[0]
    if out is None:
        out = torch.empty((M, q.rows), dtype=out_dtype, device=X.device)
    _require_out(out, M * q.rows, X.device)
    if q.device != X.device:
        raise ValueError(f"the weight is on {q.device}, X on {X.device}")
    st = q.struct()
    _check(lib().nf4_matmul_fwd(X.data_ptr(), M, ctypes.byref(st), out.data_ptr(), _dtype_enum(out.dtype),
                                _stream(X.device)), "nf4_matmul_fwd")
    return out


def nf4_matmul_bwd_dx(dY: torch.Tensor, q: QTensor, out_dtype: torch.dtype = torch.float32,
                      out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """dX = dY W^ (gradient of Y = X W^T with respect to X).  dY: bf16 [M, N] (N = q.rows)."""
    _require_device(dY, "dY")
    if dY.dtype != torch.bfloat16 or dY.dim() != 2 or dY.shape[1] != q.rows:
        raise ValueError("dY must be bf16 [M, q.rows]")
    M = dY.shape[0]
    if out is None:
        out = torch.empty((M, q.cols), dtype=out_dtype, device=dY.device)
    _require_out(out, M * q.cols, dY.device)
    if q.device != dY.device:
        raise ValueError(f"the weight is on {q.device}, dY on {dY.device}")
    st = q.struct()
    _check(lib().nf4_matmul_bwd_dx(dY.data_ptr(), M, ctypes.byref(st), out.data_ptr(), _dtype_enum(out.dtype),
                                   _stream(dY.device)), "nf4_matmul_bwd_dx")
    return out


def _lowrank_operands(U: torch.Tensor, V: torch.Tensor, M: int, cols: int, names: tuple,
                      device: torch.device) -> int:
    for t, nm in zip((U, V), names):
        _require_device(t, nm)
        if t.device != device:
            raise ValueError(f"{nm} is on {t.device}, the other operands on {device}")
        if t.dtype != torch.bfloat16 or t.dim() != 2:
            raise ValueError(f"{nm} must be a 2-D bf16 tensor")
    r = U.shape[1]
    if U.shape[0] != M or V.shape != (cols, r):
        raise ValueError(f"{names[0]} must be [{M}, r] and {names[1]} [{cols}, r] (got {tuple(U.shape)}, "
                         f"{tuple(V.shape)})")
    return r


def nf4_matmul_fwd_lora(X: torch.Tensor, q: QTensor, U: torch.Tensor, B: torch.Tensor,
                        out_dtype: torch.dtype = torch.float32, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Y = X W^T + U B^T in one fused pass.  U: bf16 [M, r] (the adapter's X A^T); B: bf16 [N, r]."""
    _require_device(X, "X")
    if X.dtype != torch.bfloat16 or X.dim() != 2 or X.shape[1] != q.cols:
        raise ValueError("X must be bf16 [M, q.cols]")
    M = X.shape[0]
    r = _lowrank_operands(U, B, M, q.rows, ("U", "B"), X.device)
    if out is None:
        out = torch.empty((M, q.rows), dtype=out_dtype, device=X.device)
    _require_out(out, M * q.rows, X.device)
    if q.device != X.device:
        raise ValueError(f"the weight is on {q.device}, X on {X.device}")
    st = q.struct()
    _check(lib().nf4_matmul_fwd_lora(X.data_ptr(), M, ctypes.byref(st), U.data_ptr(), B.data_ptr(), r,
                                     out.data_ptr(), _dtype_enum(out.dtype), _stream(X.device)),
           "nf4_matmul_fwd_lora")
    return out


def nf4_matmul_bwd_dx_lora(dY: torch.Tensor, q: QTensor, V: torch.Tensor, At: torch.Tensor,
                           out_dtype: torch.dtype = torch.float32,
                           out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """dX = dY W^ + V A in one fused pass.  V: bf16 [M, r] (dY B); At: bf16 [K, r] (A transposed)."""
    _require_device(dY, "dY")
    if dY.dtype != torch.bfloat16 or dY.dim() != 2 or dY.shape[1] != q.rows:
        raise ValueError("dY must be bf16 [M, q.rows]")
    M = dY.shape[0]
    r = _lowrank_operands(V, At, M, q.cols, ("V", "At"), dY.device)
    if out is None:
        out = torch.empty((M, q.cols), dtype=out_dtype, device=dY.device)
    _require_out(out, M * q.cols, dY.device)
    if q.device != dY.device:
        raise ValueError(f"the weight is on {q.device}, dY on {dY.device}")
    st = q.struct()
    _check(lib().nf4_matmul_bwd_dx_lora(dY.data_ptr(), M, ctypes.byref(st), V.data_ptr(), At.data_ptr(), r,
                                        out.data_ptr(), _dtype_enum(out.dtype), _stream(dY.device)),
           "nf4_matmul_bwd_dx_lora")
    return out


def _row_strided(t: torch.Tensor, name: str) -> int:
    """Row stride (elements) of a 2-D device bf16 tensor whose rows are contiguous."""
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device (HIP) tensor")
    if t.dtype != torch.bfloat16 or t.dim() != 2:
        raise ValueError(f"{name} must be a 2-D bf16 tensor")
    if t.stride(1) != 1 and t.shape[1] > 1:
        raise ValueError(f"{name} must have contiguous rows (stride 1 along its last dimension)")
    return max(t.stride(0), t.shape[1], 1)


def nf4_adapter_matmul(A: torch.Tensor, B: torch.Tensor, trans_a: bool = False, trans_b: bool = False,
                       alpha: float = 1.0, out_dtype: torch.dtype = torch.float32,
                       out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """C = alpha op(A) op(B) (the adapter's dense products), op the identity or the transpose.

    A and B are 2-D bf16 device tensors with contiguous rows; op(A) is A.T when
    ``trans_a`` (A stored [K, M]), op(B) is B.T when ``trans_b`` (B stored [N, K]).
    """
    lda, ldb = _row_strided(A, "A"), _row_strided(B, "B")
    M, K = (A.shape[1], A.shape[0]) if trans_a else (A.shape[0], A.shape[1])
    Kb, N = (B.shape[1], B.shape[0]) if trans_b else (B.shape[0], B.shape[1])
    if Kb != K:
        raise ValueError(f"op(A) is [{M}, {K}] and op(B) is [{Kb}, {N}]: reduction sizes differ")
    if A.device != B.device:
        raise ValueError(f"A is on {A.device}, B on {B.device}")
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=A.device)
    _require_out(out, M * N, A.device)
    _check(lib().nf4_adapter_matmul(int(trans_a), int(trans_b), M, N, K, float(alpha), A.data_ptr(), lda,
                                    B.data_ptr(), ldb, out.data_ptr(), _dtype_enum(out.dtype), N,
                                    _stream(A.device)), "nf4_adapter_matmul")
    return out

