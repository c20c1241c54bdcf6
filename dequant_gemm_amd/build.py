"""Builds libnf4.so (the HIP kernels and the C ABI) in-tree for gfx950.

    python -m dequant_gemm_amd.build            # compile and link
    python -m dequant_gemm_amd.build --asm DIR  # also keep the gfx950 assembly in DIR

Every compile uses hipcc with: round-to-nearest IEEE division (the quantizer's
normalisation must be the correctly rounded quotient), no floating-point
contraction (the dequantized absmax is a multiply then an add, two roundings),
and packed-fp32 instructions disabled.
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libnf4.so")
OBJDIR = os.path.join(ROOT, "_build")

SOURCES = ["nf4_api.hip", "quantize.hip", "dequantize.hip", "gemm_fwd.hip", "gemm_bwd.hip", "adapter.hip"]
# the benchmark's HBM read stream, a library of its own (include/nf4_bench.h)
BENCH_SOURCES = ["bench_stream.hip"]
BENCH_LIB = os.path.join(PKG, "libnf4_bench.so")
HEADERS = ["nf4_common.h", "nf4_launch.h"]

ARCH = "gfx950"


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    path = os.path.join(rocm, "bin", "hipcc")
    if not os.path.exists(path):
        found = shutil.which("hipcc")
        if not found:
            raise RuntimeError("hipcc not found: the ROCm toolchain is required to build libnf4")
        path = found
    return path


def compile_flags() -> list[str]:
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-fno-gpu-rdc",
        "-ffp-contract=off", "-fhip-fp32-correctly-rounded-divide-sqrt",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wno-unused-command-line-argument",
        f"-I{os.path.join(ROOT, 'include')}",
    ]


def _compile(src: str, asm_dir: str | None, objdir=None) -> str:
    obj = os.path.join(objdir or OBJDIR, os.path.splitext(src)[0] + ".o")
    _run([hipcc(), *compile_flags(), "-c", os.path.join(CSRC, src), "-o", obj])
    if asm_dir:
        os.makedirs(asm_dir, exist_ok=True)
        out = os.path.join(asm_dir, os.path.splitext(src)[0] + f"-{ARCH}.s")
        _run([hipcc(), *compile_flags(), "--cuda-device-only", "-S", os.path.join(CSRC, src), "-o", out])
    return obj


def _run(cmd):
    p = subprocess.run(cmd, capture_output=True, text=True)
    noise = ("is not a recognized feature for this target", "ignoring feature")
    errs = "\n".join(l for l in (p.stderr or "").splitlines() if not any(n in l for n in noise))
    if p.returncode != 0:
        raise RuntimeError(f"command failed ({p.returncode}): {' '.join(cmd)}\n{errs}")
    if errs.strip():
        sys.stderr.write(errs + "\n")


def build(asm_dir: str | None = None, verbose: bool = True) -> str:
    """Compiles every source and links libnf4.so (and the benchmark's libnf4_bench.so); returns
    the path of libnf4.so."""
    lib = LIB
    os.makedirs(OBJDIR, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES + BENCH_SOURCES), os.cpu_count() or 1)) as ex:
        objs = list(ex.map(lambda s: _compile(s, asm_dir), SOURCES + BENCH_SOURCES))
    for out, part in ((lib, objs[:len(SOURCES)]), (BENCH_LIB, objs[len(SOURCES):])):
        tmp = out + ".tmp"
        _run([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *part])
        os.replace(tmp, out)
    if verbose:
        print(f"built {lib}")
    return lib


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--asm", default=None, help="directory for the gfx950 assembly listings")
    a = ap.parse_args()
    build(a.asm)
