"""The C ABI's validation paths under AddressSanitizer and UndefinedBehaviorSanitizer.

The host code of the API (nf4_api.hip) is compiled with both sanitizers and
linked, with the kernels built as usual, into a small C driver
(tests/asan/abi_driver.c) that forces every documented error code and calls
the host-only functions.  None of these paths reaches a HIP call, so this runs
on a machine without a GPU.  The sanitizers apply to host code only.
"""
import os
import subprocess

import pytest

from dequant_gemm_amd import build as B

HERE = os.path.dirname(os.path.abspath(__file__))


def _have_hipcc() -> bool:
    try:
        return os.path.exists(B.hipcc())
    except RuntimeError:
        return False


def _kernel_objects(objdir):
    """The kernels' objects from the in-tree build when they are newer than every source and
    header, else compiled afresh into ``objdir``."""
    newest = max(os.path.getmtime(os.path.join(B.CSRC, f)) for f in B.SOURCES + B.HEADERS)
    newest = max(newest, os.path.getmtime(os.path.join(B.ROOT, "include", "nf4.h")))
    out = []
    for src in B.SOURCES:
        if src == "nf4_api.hip":
            continue
        obj = os.path.join(B.OBJDIR, os.path.splitext(src)[0] + ".o")
        out.append(obj if os.path.exists(obj) and os.path.getmtime(obj) >= newest else B._compile(src, None, objdir))
    return out


@pytest.mark.skipif(not _have_hipcc(), reason="hipcc not found")
def test_validation_paths_are_clean_under_sanitizers(tmp_path):
    objdir = str(tmp_path)
    kernels = _kernel_objects(objdir)
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
    api = os.path.join(objdir, "nf4_api_san.o")
    subprocess.run([B.hipcc(), *B.compile_flags(), *san, "-c", os.path.join(B.CSRC, "nf4_api.hip"), "-o", api],
                   check=True, capture_output=True)
    exe = os.path.join(objdir, "abi_driver")
    subprocess.run([B.hipcc(), f"--offload-arch={B.ARCH}", *san, f"-I{os.path.join(B.ROOT, 'include')}",
                    "-x", "c", os.path.join(HERE, "asan", "abi_driver.c"), "-x", "none", api, *kernels,
                    "-o", exe], check=True, capture_output=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0, r.stderr[-4000:]
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr[-4000:]
