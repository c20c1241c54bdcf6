"""The backward kernels' transposing LDS reads, checked in their gfx950 assembly (CPU only).

The wide backward kernel issues ``ds_read_b64_tr_b16`` as inline assembly (the
compiler's wait insertion would otherwise wait for every buffer-to-LDS load in
flight before each such read) and waits for the results itself.  The compiler
takes an inline-asm result as written as soon as the statement is issued, so two
mistakes stay invisible to it: a result that nothing consumes (its registers are
then free for reuse while the load is still in flight, and the late data lands on
whatever was put there), and a use of a result before a wait that covers the
load.  This test compiles gemm_bwd.hip to assembly with the library's own flags
and checks, for every transposing read of every backward kernel, that the first
later instruction that reads or writes one of its destination registers comes
after an ``s_waitcnt lgkmcnt(n)`` with at most n LDS instructions issued between
the read and the wait.  No GPU is needed; hipcc cross-compiles.
"""
import os
import re
import shutil
import subprocess

import pytest

from dequant_gemm_amd import build as B

pytestmark = pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
                                reason="needs hipcc (ROCm) to compile the kernels to assembly")


def _regs(text):
    out = set()
    for m in re.finditer(r"\bv\[(\d+):(\d+)\]", text):
        out |= set(range(int(m.group(1)), int(m.group(2)) + 1))
    for m in re.finditer(r"\bv(\d+)\b", text):
        out.add(int(m.group(1)))
    return out


def unprotected_tr_reads(asm_lines):
    """(read line, use line) pairs where a transposing read's destination is touched before a covering wait."""
    lines = [l.split(";")[0].strip() for l in asm_lines]
    bad = []
    for i, l in enumerate(lines):
        if not l.startswith("ds_read_b64_tr_b16"):
            continue
        dst = _regs(l.split(None, 1)[1].split(",")[0])
        later_lds = 0
        for k in range(i + 1, len(lines)):
            t = lines[k]
            if not t or t.startswith(".") or t.endswith(":"):
                continue
            if t.startswith("s_endpgm"):
                break
            m = re.match(r"s_waitcnt\b.*lgkmcnt\((\d+)\)", t)
            if m and int(m.group(1)) <= later_lds:
                break
            ops = t.split(None, 1)
            if len(ops) == 2 and not t.startswith("s_waitcnt") and _regs(ops[1]) & dst:
                bad.append((i + 1, k + 1, l, t))
                break
            if t.startswith("ds_"):
                later_lds += 1
    return bad


def _kernels(asm_text, name):
    src = asm_text.split("\n")
    starts = [i for i, l in enumerate(src) if re.match(r"^_Z\S*" + name + r"\S*:", l)]
    for s in starts:
        e = s
        while e < len(src) and "s_endpgm" not in src[e]:
            e += 1
        yield src[s].split(":")[0], src[s:e + 1]


def test_checker_flags_a_use_before_the_wait():
    # a planted mistake in a hand-written listing: the destination is read before any wait
    listing = ["ds_read_b64_tr_b16 v[2:3], v90 offset:0", "v_mov_b32_e32 v5, v2", "s_waitcnt lgkmcnt(0)",
               "s_endpgm"]
    assert len(unprotected_tr_reads(listing)) == 1
    # a wait that allows the read itself to be outstanding does not cover it
    listing = ["ds_read_b64_tr_b16 v[2:3], v90 offset:0", "ds_read_b128 v[8:11], v91", "s_waitcnt lgkmcnt(2)",
               "v_mov_b32_e32 v5, v3", "s_endpgm"]
    assert len(unprotected_tr_reads(listing)) == 1
    # covered: one later LDS instruction, lgkmcnt(1)
    listing = ["ds_read_b64_tr_b16 v[2:3], v90 offset:0", "ds_read_b128 v[8:11], v91", "s_waitcnt lgkmcnt(1)",
               "v_mov_b32_e32 v5, v3", "s_endpgm"]
    assert unprotected_tr_reads(listing) == []
    # a later read into the same registers before the wait is a use too
    listing = ["ds_read_b64_tr_b16 v[2:3], v90 offset:0", "ds_read_b64_tr_b16 v[2:3], v90 offset:64",
               "s_waitcnt lgkmcnt(0)", "s_endpgm"]
    assert len(unprotected_tr_reads(listing)) == 1


def test_backward_transposing_reads_are_waited_for(tmp_path):
    out = tmp_path / "gemm_bwd.s"
    cmd = [B.hipcc(), *B.compile_flags(), "--cuda-device-only", "-S", os.path.join(B.CSRC, "gemm_bwd.hip"),
           "-o", str(out)]
    p = subprocess.run(cmd, capture_output=True, text=True)
    assert p.returncode == 0, p.stderr[-2000:]
    text = out.read_text()
    kernels = list(_kernels(text, "bwd_dx_wide_kernel"))
    assert len(kernels) == 32, "every instantiation of the wide backward kernel"
    n_reads = 0
    for name, lines in kernels:
        n_reads += sum(1 for l in lines if l.strip().startswith("ds_read_b64_tr_b16"))
        bad = unprotected_tr_reads(lines)
        assert not bad, f"{name}: transposing read used before its wait: {bad[:3]}"
    assert n_reads > 0
