"""Seeded synthetic inputs for the NF4 quantize and dequant-GEMM workloads.

This module only draws random numbers and lays them out; it holds none of the
quantization or matrix-product arithmetic, so the CPU oracle and the GPU path
can both take their inputs from here without sharing any of the method.

Recipe (every tensor):
  * ``numpy.random.Generator(PCG64(seed))``;
  * ``standard_normal`` in float64 times the standard deviation, or
    ``standard_t(nu)`` times a scale, drawn in chunks of ``_CHUNK`` values in
    row-major order (the chunking does not change the stream);
  * the float64 product rounded to float32 (round-to-nearest-even, numpy's
    unsafe cast on output), and from there to bfloat16 by torch's conversion
    (round-to-nearest-even) where the workload calls for bf16.

Workloads and seeds (``N(0, s)`` means standard deviation ``s``):
  tiny     W [256,256] f32 N(0,0.02) seed 0; X [8,256] bf16 N(0,1) seed 1;
           dY [8,256] bf16 N(0,1) seed 2
  decode   W [4096,4096] bf16 N(0,0.02), a pool of independently seeded
           weights, seed 1000+p; X [M,4096] bf16 N(0,1) seed 1100+M
  prefill  W [11008,4096] bf16 N(0,0.02) seed 2000; X [4096,4096] bf16 N(0,1)
           seed 2001; dY [4096,11008] bf16 N(0,0.01) seed 2002
  bulk     32 decoder layers, d=4096, ffn=11008; per layer the matrices
           q,k,v,o [4096,4096], gate,up [11008,4096], down [4096,11008]
           (stored [out,in]), bf16 N(0,0.02), seed 3000+7*layer+j
  large    W [28672,8192] f32 0.02*t(nu=4) seed 4000; X [8192,8192] bf16
           N(0,1) seed 4001; dY [8192,28672] bf16 N(0,0.01) seed 4002
"""
from __future__ import annotations

import concurrent.futures as _cf
import os

import numpy as np
import torch

_CHUNK = 1 << 20

BULK_LAYERS = 32
BULK_D = 4096
BULK_FFN = 11008
BULK_NAMES = ("q", "k", "v", "o", "gate", "up", "down")


def _draw(kind: str, n: int, seed: int, scale: float, df: float = 4.0) -> np.ndarray:
    rng = np.random.Generator(np.random.PCG64(seed))
    out = np.empty(n, dtype=np.float32)
    tmp = np.empty(min(_CHUNK, n), dtype=np.float64)
    for lo in range(0, n, _CHUNK):
        m = min(_CHUNK, n - lo)
        if kind == "normal":
            v = rng.standard_normal(out=tmp[:m])
        elif kind == "t":
            v = rng.standard_t(df, m)
        else:
            raise ValueError(kind)
        # float64 product rounded to float32 (nearest-even) on the way out
        np.multiply(v, scale, out=out[lo:lo + m], casting="unsafe")
    return out


def tensor(kind: str, shape, seed: int, scale: float, dtype: torch.dtype, df: float = 4.0) -> torch.Tensor:
    """A CPU tensor of ``shape`` drawn per the module recipe, in ``dtype``."""
    n = 1
    for s in shape:
        n *= int(s)
    f32 = torch.from_numpy(_draw(kind, n, seed, scale, df)).reshape(tuple(shape))
    if dtype == torch.float32:
        return f32
    if dtype == torch.bfloat16:
        return f32.to(torch.bfloat16)
    raise ValueError(dtype)


def normal(shape, std: float, seed: int, dtype: torch.dtype = torch.bfloat16) -> torch.Tensor:
    return tensor("normal", shape, seed, std, dtype)


def student_t(shape, df: float, scale: float, seed: int, dtype: torch.dtype = torch.float32) -> torch.Tensor:
    return tensor("t", shape, seed, scale, dtype, df=df)


# ---------------------------------------------------------------- workloads

def tiny():
    """Tiny: W 256x256 fp32, X and dY 8x256 bf16."""
    return {
        "W": normal((256, 256), 0.02, 0, torch.float32),
        "X": normal((8, 256), 1.0, 1),
        "dY": normal((8, 256), 1.0, 2),
    }


DECODE_K = 4096
DECODE_N = 4096
DECODE_MS = (1, 4, 16)


def decode_weight(p: int) -> torch.Tensor:
    return normal((DECODE_N, DECODE_K), 0.02, 1000 + p)


def decode_x(m: int) -> torch.Tensor:
    return normal((m, DECODE_K), 1.0, 1100 + m)


PREFILL_M, PREFILL_K, PREFILL_N = 4096, 4096, 11008


def prefill_weight() -> torch.Tensor:
    return normal((PREFILL_N, PREFILL_K), 0.02, 2000)


def prefill_x() -> torch.Tensor:
    return normal((PREFILL_M, PREFILL_K), 1.0, 2001)


def prefill_dy() -> torch.Tensor:
    return normal((PREFILL_M, PREFILL_N), 0.01, 2002)


LARGE_M, LARGE_K, LARGE_N = 8192, 8192, 28672


def large_weight() -> torch.Tensor:
    return student_t((LARGE_N, LARGE_K), 4.0, 0.02, 4000)


def large_x() -> torch.Tensor:
    return normal((LARGE_M, LARGE_K), 1.0, 4001)


def large_dy() -> torch.Tensor:
    return normal((LARGE_M, LARGE_N), 0.01, 4002)


def bulk_shape(j: int):
    name = BULK_NAMES[j]
    if name in ("q", "k", "v", "o"):
        return (BULK_D, BULK_D)
    if name in ("gate", "up"):
        return (BULK_FFN, BULK_D)
    return (BULK_D, BULK_FFN)


def bulk_weight(layer: int, j: int) -> torch.Tensor:
    return normal(bulk_shape(j), 0.02, 3000 + 7 * layer + j)


def parallel(fn, args, workers: int | None = None):
    """[fn(a) for a in args], drawn on a thread pool (numpy's generators release the GIL)."""
    args = list(args)
    if workers is None:
        workers = min(16, len(os.sched_getaffinity(0)))
    with _cf.ThreadPoolExecutor(max_workers=max(1, workers)) as ex:
        return list(ex.map(fn, args))


def bulk_weights_parallel(keys, workers: int | None = None):
    """Several bulk matrices at once; ``keys`` are (layer, j); returns a dict keyed the same way."""
    keys = list(keys)
    return dict(zip(keys, parallel(lambda k: bulk_weight(*k), keys, workers)))
