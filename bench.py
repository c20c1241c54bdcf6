"""Benchmark of the NF4 hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
                    [--no-decode] [--no-large] [--no-bulk] [--op OP]

One step is one training-layer pass of the prefill workload (X [4096,4096]
bf16, weight [11008,4096] bf16 N(0,0.02), dY [4096,11008] bf16 N(0,0.01)):
NF4 quantization with double quantization of the weight, the fused forward
Y = X W^T and the fused backward dX = dY W^, all through the C ABI of
libnf4.so on torch's current stream, inputs and outputs resident in HBM.

``value`` is the step's GEMM throughput, 2 * 2*M*N*K flops per step over the
step time (quantization included in the time; the timed steps run back to back
with events only at the two ends).  The same JSON line carries per-kernel
timings (HIP events around every launch of a second pass of as many steps), the
dequantizer, the rank-64 adapter variants of both GEMMs, the decode-shape
forward (M = 1, 4, 16 on a rotating pool of 512 quantized 4096x4096 weights,
replayed from a HIP graph so host launch overhead does not count; and each
dispatch's own duration from a rocprofv3 kernel trace of a child process), the
backward dX = dY W^ at the same row counts over the same pool, a
plain HBM read stream (the achievable bandwidth), the
outlier-heavy large shape (M = K = 8192, N = 28672, fp32 Student-t weight), the
32-layer bulk quantize/dequantize round trip, the prefill workload at block sizes
32, 128 and 256, a roofline entry for the dominant
kernel and the CPU oracle's throughput on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "NF4 dequant-GEMM TFLOP/s + GB/s (fwd, bwd-dX) and % of MFMA/HBM roofline"
PEAK_BF16_TFLOPS = 2516.6   # 256 CU x 2.4 GHz x 4096 flop/clk (the published 2.5 PF dense)
PEAK_HBM_GBPS = 8000.0      # HBM3E


def _code_only(text: str) -> str:
    """C++ source with comments and blank lines removed and spaces at line ends trimmed."""
    import re
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    return "\n".join(l.rstrip() for l in text.splitlines() if l.strip())


def _source_hash(files):
    """Hash of the kernels' code (comments excluded, so a comment edit keeps counters valid)."""
    import hashlib
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, f), encoding="utf-8") as fh:
            h.update(_code_only(fh.read()).encode())
    return h.hexdigest()[:16]


def measured_traffic(kernel):
    """HBM-side bytes per launch from the committed counter summary, or None.

    ``profiles/traffic.json`` records, per kernel, FETCH_SIZE and WRITE_SIZE scaled by
    a plain-copy calibration and the hash of the kernel's sources when the counters were
    taken; a changed source makes the figure stale and it is not reported.
    """
    try:
        with open(os.path.join(ROOT, "profiles", "traffic.json")) as fh:
            ent = json.load(fh)["kernels"].get(kernel)
        if ent and ent["source_sha256"] == _source_hash(ent["sources"]):
            return ent["bytes_per_launch"]
    except (OSError, KeyError, ValueError):
        pass
    return None


# kernels whose HBM-side traffic is recorded: kernel name -> (profiling op, source files)
TRAFFIC_KERNELS = {
    "fwd_wide_kernel": ("fwd", ["dequant_gemm_amd/csrc/gemm_fwd.hip", "dequant_gemm_amd/csrc/nf4_common.h"]),
    "bwd_dx_wide_kernel": ("bwd_dx", ["dequant_gemm_amd/csrc/gemm_bwd.hip", "dequant_gemm_amd/csrc/nf4_common.h"]),
}
COPY_BYTES = 1 << 30   # the calibration copy of run_single_op("copy")


def write_traffic(pmc_dir):
    """Write profiles/traffic.json from rocprofv3 counter runs (never by hand).

    ``pmc_dir`` holds the CSV output of ``rocprofv3 --pmc FETCH_SIZE`` and ``--pmc WRITE_SIZE``
    (one counter per run) of ``bench.py --op <op>`` for op = copy and each op in
    TRAFFIC_KERNELS, in ``pmc_<COUNTER>_<op>/<op>_counter_collection.csv``.  The per-dispatch
    KiB of each kernel (mean over its dispatches) are scaled by what the same counter reads
    for the plain 1 GiB copy, and stored with the hash of the kernel's sources.
    """
    import csv

    def mean_kib(counter, op, name):
        f = os.path.join(pmc_dir, f"pmc_{counter}_{op}", f"{op}_counter_collection.csv")
        per = {}
        with open(f, newline="") as fh:
            for r in csv.DictReader(fh):
                if r["Counter_Name"] == counter and name in r["Kernel_Name"]:
                    per[r["Dispatch_Id"]] = per.get(r["Dispatch_Id"], 0.0) + float(r["Counter_Value"])
        if not per:
            raise ValueError(f"no {counter} rows for {name} in {f}")
        return sum(per.values()) / len(per), len(per)

    cf, _ = mean_kib("FETCH_SIZE", "copy", "copyBuffer")
    cw, _ = mean_kib("WRITE_SIZE", "copy", "copyBuffer")
    ff, wf = COPY_BYTES / 1024 / cf, COPY_BYTES / 1024 / cw
    out = {"calibration": {"copy_bytes": COPY_BYTES, "fetch_factor": round(ff, 4), "write_factor": round(wf, 4)},
           "command": "rocprofv3 --pmc FETCH_SIZE (then WRITE_SIZE) --output-format csv -- "
                      "python3 bench.py --op <op> --steps 4 --warmup 1",
           "kernels": {}}
    for name, (op, files) in TRAFFIC_KERNELS.items():
        fk, n1 = mean_kib("FETCH_SIZE", op, name)
        wk, n2 = mean_kib("WRITE_SIZE", op, name)
        fb, wb = int(fk * 1024 * ff), int(wk * 1024 * wf)
        out["kernels"][name] = {"op": op, "sources": files, "source_sha256": _source_hash(files),
                                "fetch_kib": round(fk, 1), "write_kib": round(wk, 1), "dispatches": [n1, n2],
                                "fetch_bytes": fb, "write_bytes": wb, "bytes_per_launch": fb + wb}
    with open(os.path.join(ROOT, "profiles", "traffic.json"), "w") as fh:
        json.dump(out, fh, indent=1)
        fh.write("\n")
    return out


def wq_bytes(rows, cols):
    numel = rows * cols
    nb = -(-numel // 64)
    return -(-numel // 2) + nb + 4 * (-(-nb // 256)) + 4


def time_graph(fn, reps, per_graph=20):
    """Average milliseconds per call of ``fn`` replayed from a HIP graph of ``per_graph`` calls.

    For kernels shorter than the host's per-call launch cost (tens of microseconds
    through ctypes), back-to-back eager calls would time the host, not the kernel.
    """
    fn()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(per_graph):
            fn()
    g.replay()
    torch.cuda.synchronize()
    ms = time_events(g.replay, reps) / per_graph
    del g
    return ms


def time_events(fn, reps, stream=None):
    """Average milliseconds of ``fn`` over ``reps`` calls between two HIP events."""
    s = torch.cuda.Event(enable_timing=True)
    e = torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(reps):
        fn()
    e.record()
    e.synchronize()
    return s.elapsed_time(e) / reps


def bench_prefill(dg, steps, warmup):
    import synth
    d = torch.device("cuda:0")
    M, K, N = synth.PREFILL_M, synth.PREFILL_K, synth.PREFILL_N
    W = synth.prefill_weight().to(d)
    X = synth.prefill_x().to(d)
    dY = synth.prefill_dy().to(d)
    q = dg.empty_qtensor(N, K, True, d)
    ws = torch.empty(dg.nf4_sizes(N, K)["workspace_bytes"], dtype=torch.uint8, device=d)
    Y = torch.empty((M, N), dtype=torch.float32, device=d)
    dX = torch.empty((M, K), dtype=torch.float32, device=d)

    ops = ("quantize", "fwd", "bwd_dx")
    ev = {o: [] for o in ops}

    def step(record):
        marks = [torch.cuda.Event(enable_timing=True) for _ in range(4)] if record else None
        if record:
            marks[0].record()
        dg.nf4_quantize(W, out=q, workspace=ws)
        if record:
            marks[1].record()
        dg.nf4_matmul_fwd(X, q, out=Y)
        if record:
            marks[2].record()
        dg.nf4_matmul_bwd_dx(dY, q, out=dX)
        if record:
            marks[3].record()
        return marks

    for _ in range(warmup):
        step(False)
    torch.cuda.synchronize()
    # The step time: exactly ``steps`` steps between two events, nothing else in
    # the stream (events between the launches cost ~4 us each, ~2% of a step).
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(steps):
        step(False)
    t1.record()
    torch.cuda.synchronize()
    ms_step = t0.elapsed_time(t1) / steps
    # Per-kernel durations: the same steps again, every launch bracketed by events.
    rec = [step(True) for _ in range(steps)]
    torch.cuda.synchronize()
    for marks in rec:
        for i, o in enumerate(ops):
            ev[o].append(marks[i].elapsed_time(marks[i + 1]))
    per = {o: float(np.mean(v)) for o, v in ev.items()}
    flop = 2.0 * M * N * K
    bytes_fwd = M * K * 2 + wq_bytes(N, K) + M * N * 4
    bytes_bwd = M * N * 2 + wq_bytes(N, K) + M * K * 4
    bytes_q = N * K * 2 + wq_bytes(N, K)
    res = {
        "ms_per_step": ms_step,
        "tflops_step": 2 * flop / (ms_step * 1e-3) / 1e12,
        "ops": {
            "quantize": {"ms": per["quantize"], "GB/s": bytes_q / (per["quantize"] * 1e-3) / 1e9},
            "fwd": {"ms": per["fwd"], "TFLOP/s": flop / (per["fwd"] * 1e-3) / 1e12,
                    "GB/s": bytes_fwd / (per["fwd"] * 1e-3) / 1e9},
            "bwd_dx": {"ms": per["bwd_dx"], "TFLOP/s": flop / (per["bwd_dx"] * 1e-3) / 1e12,
                       "GB/s": bytes_bwd / (per["bwd_dx"] * 1e-3) / 1e9},
        },
        "flop_per_gemm": flop,
    }
    for o in ("fwd", "bwd_dx"):
        res["ops"][o]["frac_mfma"] = res["ops"][o]["TFLOP/s"] / PEAK_BF16_TFLOPS
    res["ops"]["quantize"]["frac_hbm"] = res["ops"]["quantize"]["GB/s"] / PEAK_HBM_GBPS

    # dequantize (context: the unfused path's first half)
    Wh = torch.empty((N, K), dtype=torch.bfloat16, device=d)
    ms_dq = time_graph(lambda: dg.nf4_dequantize(q, out=Wh), 10)
    bdq = wq_bytes(N, K) + N * K * 2
    res["ops"]["dequantize"] = {"ms": ms_dq, "GB/s": bdq / (ms_dq * 1e-3) / 1e9,
                                "frac_hbm": bdq / (ms_dq * 1e-3) / 1e9 / PEAK_HBM_GBPS}
    # the naive dequantize-then-multiply the pages compare against, for context
    naive = lambda: (dg.nf4_dequantize(q, out=Wh), torch.matmul(X, Wh.t()))
    for _ in range(3):          # library load and kernel selection happen on the first calls
        naive()
    torch.cuda.synchronize()
    ms_naive = time_events(naive, 10)
    res["ops"]["naive_dequant_then_matmul_fwd"] = {"ms": ms_naive, "TFLOP/s": flop / (ms_naive * 1e-3) / 1e12}
    res["ops"].update(_dense_gemm_reference(X, dY, Wh, flop))
    # the same GEMMs with a rank-64 low-rank adapter term fused in (U, B / V, A^T bf16)
    r = 64
    U = synth.normal((M, r), 1.0, 2100).to(d)
    Bl = synth.normal((N, r), 0.1, 2101).to(d)
    V = synth.normal((M, r), 1.0, 2102).to(d)
    At = synth.normal((K, r), 0.1, 2103).to(d)
    # The clock drifts by several percent between back-to-back measurements under
    # these power-limited kernels, so each variant is timed interleaved with the
    # plain call and compared by the ratio of medians.
    for name, fn, plain, base in (
            ("fwd_lora_r64", lambda: dg.nf4_matmul_fwd_lora(X, q, U, Bl, out=Y),
             lambda: dg.nf4_matmul_fwd(X, q, out=Y), "fwd"),
            ("bwd_dx_lora_r64", lambda: dg.nf4_matmul_bwd_dx_lora(dY, q, V, At, out=dX),
             lambda: dg.nf4_matmul_bwd_dx(dY, q, out=dX), "bwd_dx")):
        fn()
        torch.cuda.synchronize()
        t_l, t_p = [], []
        for _ in range(5):
            t_p.append(time_events(plain, 4))
            t_l.append(time_events(fn, 4))
        ms_l, ms_p = float(np.median(t_l)), float(np.median(t_p))
        fl = flop + 2.0 * M * (N if base == "fwd" else K) * r
        res["ops"][name] = {"ms": ms_l, "TFLOP/s": fl / (ms_l * 1e-3) / 1e12,
                            "time_vs_plain": ms_l / ms_p}
    del U, Bl, V, At
    del W, X, dY, Y, dX, Wh, ws
    return res


def bench_decode(dg, pool=512, reps=10):
    import synth
    d = torch.device("cuda:0")
    K, N = synth.DECODE_K, synth.DECODE_N
    # a pool of 512 independently seeded quantized weights (4.4 GB, 17x the 256 MB
    # last-level cache), N(0, 0.02) drawn on the device with seed 1000 + p, rotated
    # call by call.  The kernel's code loads are non-temporal; under a cyclic pool
    # they leave part of the last-level cache holding earlier weights, so the pool
    # is large enough that such hits are a few percent of the bytes.
    qs = []
    for p in range(pool):
        qs.append(dg.nf4_quantize(_device_normal((N, K), 0.02, 1000 + p, d)))
    torch.cuda.synchronize()
    out = {}
    for M in synth.DECODE_MS:
        X = synth.decode_x(M).to(d)
        Y = torch.empty((M, N), dtype=torch.float32, device=d)
        for qq in qs:
            dg.nf4_matmul_fwd(X, qq, out=Y)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for qq in qs:
                dg.nf4_matmul_fwd(X, qq, out=Y)
        g.replay()
        torch.cuda.synchronize()
        ms = time_events(g.replay, reps) / pool
        b = M * K * 2 + wq_bytes(N, K) + M * N * 4
        out[f"decode_m{M}"] = {"us": ms * 1e3, "GB/s": b / (ms * 1e-3) / 1e9,
                               "frac_hbm": b / (ms * 1e-3) / 1e9 / PEAK_HBM_GBPS,
                               "TFLOP/s": 2.0 * M * N * K / (ms * 1e-3) / 1e12}
        del g
        # the backward dX = dY W^ at the same row counts over the same pool (context:
        # a small-batch backward, one workgroup per 32 output columns streaming the weight)
        dY = _device_normal((M, N), 1.0, 1200 + M, d)
        dX = torch.empty((M, K), dtype=torch.float32, device=d)
        for qq in qs:
            dg.nf4_matmul_bwd_dx(dY, qq, out=dX)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for qq in qs:
                dg.nf4_matmul_bwd_dx(dY, qq, out=dX)
        g.replay()
        torch.cuda.synchronize()
        ms = time_events(g.replay, reps) / pool
        b = M * N * 2 + wq_bytes(N, K) + M * K * 4
        out[f"decode_bwd_dx_m{M}"] = {"us": ms * 1e3, "GB/s": b / (ms * 1e-3) / 1e9,
                                      "frac_hbm": b / (ms * 1e-3) / 1e9 / PEAK_HBM_GBPS}
        del g, dY, dX
    # Context: the per-call floor of this measurement -- a one-element kernel replayed
    # the same way (one launch per pool entry).  No kernel can take less per call here.
    t = torch.zeros(1, device=d)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(pool):
            t.add_(1.0)
    g.replay()
    torch.cuda.synchronize()
    out["decode_launch_floor"] = {"us": time_events(g.replay, reps) / pool * 1e3,
                                  "what": f"one-element kernel, {pool} per HIP graph, per call"}
    return out


def _dense_gemm_reference(X, dY, Wh, flop, reps=10):
    """Context for the matrix-core bar: the platform's own dense bf16 GEMM (hipBLASLt through
    torch.matmul, bf16 in and out) on the same shapes with the weight already dense bf16, in
    the faster of two weight layouts (as stored [N, K], and transposed to [K, N])."""
    Wt = Wh.t().contiguous()
    cands = {"fwd": [lambda: torch.matmul(X, Wh.t()), lambda: torch.matmul(X, Wt)],
             "bwd_dx": [lambda: torch.matmul(dY, Wh), lambda: torch.matmul(dY, Wt.t())]}
    out = {}
    for name, fns in cands.items():
        best = None
        for fn in fns:
            for _ in range(3):
                fn()
            torch.cuda.synchronize()
            ms = time_events(fn, reps)
            best = ms if best is None else min(best, ms)
        tf = flop / (best * 1e-3) / 1e12
        out[f"dense_bf16_{name}_hipblaslt"] = {"ms": best, "TFLOP/s": tf, "frac_mfma": tf / PEAK_BF16_TFLOPS}
    del Wt
    return out


def _device_normal(shape, std, seed, d, dtype=torch.bfloat16):
    g = torch.Generator(device=d)
    g.manual_seed(seed)
    return (torch.randn(shape, generator=g, device=d, dtype=torch.float32) * std).to(dtype)


def bench_large(dg, reps=5):
    """The outlier-heavy large shape: M=8192, K=8192, N=28672, W = 0.02 * Student-t(4) fp32.

    Inputs are drawn on the device (seeded torch generators, the workload's shapes and
    distributions); the parity tests draw the same workload on the host.
    """
    import synth
    d = torch.device("cuda:0")
    M, K, N = synth.LARGE_M, synth.LARGE_K, synth.LARGE_N
    torch.manual_seed(4000)
    W = (torch.distributions.StudentT(torch.tensor(4.0, device=d)).sample((N, K)) * 0.02).float().contiguous()
    X = _device_normal((M, K), 1.0, 4001, d)
    dY = _device_normal((M, N), 0.01, 4002, d)
    q = dg.empty_qtensor(N, K, True, d)
    ws = torch.empty(dg.nf4_sizes(N, K)["workspace_bytes"], dtype=torch.uint8, device=d)
    Y = torch.empty((M, N), dtype=torch.float32, device=d)
    dX = torch.empty((M, K), dtype=torch.float32, device=d)
    quant = lambda: dg.nf4_quantize(W, out=q, workspace=ws)
    quant()
    torch.cuda.synchronize()
    ms_q = time_events(quant, reps)
    fwd = lambda: dg.nf4_matmul_fwd(X, q, out=Y)
    bwd = lambda: dg.nf4_matmul_bwd_dx(dY, q, out=dX)
    fwd(), bwd()
    torch.cuda.synchronize()
    ms_f = time_events(fwd, reps)
    ms_b = time_events(bwd, reps)
    flop = 2.0 * M * N * K
    dec = _large_decode(dg, q, X, W, ws, reps)
    bq = N * K * 4 + wq_bytes(N, K)
    out = {"large_quantize_f32": {"ms": ms_q, "GB/s": bq / (ms_q * 1e-3) / 1e9,
                                  "frac_hbm": bq / (ms_q * 1e-3) / 1e9 / PEAK_HBM_GBPS}}
    for name, ms in (("large_fwd", ms_f), ("large_bwd_dx", ms_b)):
        tf = flop / (ms * 1e-3) / 1e12
        out[name] = {"ms": ms, "TFLOP/s": tf, "frac_mfma": tf / PEAK_BF16_TFLOPS}
    out.update(dec)
    Wh = dg.nf4_dequantize(q)
    out.update({"large_" + k: v for k, v in _dense_gemm_reference(X, dY, Wh, flop, reps).items()})
    del W, X, dY, q, ws, Y, dX, Wh
    torch.cuda.empty_cache()
    return out


LARGE_DECODE_COPIES = 3       # 3 x 121 MB rotating: more than the 256 MB last-level cache


def _large_decode(dg, q, X, W, ws, reps, rounds=8):
    """Decode (M = 1, 4, 16: the first rows of X) on the 28672 x 8192 weight: three quantized
    copies rotating call by call, one HIP graph of ``rounds`` passes over them, per call."""
    import synth
    d = X.device
    N, K = q.rows, q.cols
    qs = [q] + [dg.nf4_quantize(W, out=dg.empty_qtensor(N, K, True, d), workspace=ws)
                for _ in range(LARGE_DECODE_COPIES - 1)]
    out = {}
    for M in synth.DECODE_MS:
        Xm = X[:M].contiguous()
        Y = torch.empty((M, N), dtype=torch.float32, device=d)
        for qq in qs:
            dg.nf4_matmul_fwd(Xm, qq, out=Y)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(rounds):
                for qq in qs:
                    dg.nf4_matmul_fwd(Xm, qq, out=Y)
        g.replay()
        torch.cuda.synchronize()
        us = time_events(g.replay, reps) / (rounds * len(qs)) * 1e3
        b = M * K * 2 + wq_bytes(N, K) + M * N * 4
        out[f"large_decode_m{M}"] = {"us": us, "GB/s": b / (us * 1e-6) / 1e9,
                                     "frac_hbm": b / (us * 1e-6) / 1e9 / PEAK_HBM_GBPS}
        del g
    del qs
    return out


def bench_bulk(dg, reps=3):
    """Bulk quantize + dequantize round trip of a 32-layer decoder's linear weights.

    Per layer q, k, v, o [4096, 4096], gate, up [11008, 4096], down [4096, 11008], bf16
    N(0, 0.02) drawn on the device (seeded per matrix); all 224 matrices are quantized, then
    all are dequantized, each pass replayed from a HIP graph.
    """
    import synth
    d = torch.device("cuda:0")
    Ws, qs = [], []
    for layer in range(synth.BULK_LAYERS):
        for j in range(len(synth.BULK_NAMES)):
            shape = synth.bulk_shape(j)
            Ws.append(_device_normal(shape, 0.02, 3000 + 7 * layer + j, d))
            qs.append(dg.empty_qtensor(shape[0], shape[1], True, d))
    numel = sum(w.numel() for w in Ws)
    ws = torch.empty(max(dg.nf4_sizes(*w.shape)["workspace_bytes"] for w in Ws), dtype=torch.uint8, device=d)
    outs = {}
    for w in Ws:
        outs.setdefault(tuple(w.shape), torch.empty(w.shape, dtype=torch.bfloat16, device=d))
    quant_all = lambda: [dg.nf4_quantize(w, out=q, workspace=ws) for w, q in zip(Ws, qs)]
    deq_all = lambda: [dg.nf4_dequantize(q, out=outs[(q.rows, q.cols)]) for q in qs]
    res = {}
    for name, fn in (("bulk_quantize", quant_all), ("bulk_dequantize", deq_all)):
        fn()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fn()
        g.replay()
        torch.cuda.synchronize()
        ms = time_events(g.replay, reps)
        b = sum(2 * w.numel() + wq_bytes(*w.shape) for w in Ws)
        res[name] = {"ms": ms, "GB/s": b / (ms * 1e-3) / 1e9, "frac_hbm": b / (ms * 1e-3) / 1e9 / PEAK_HBM_GBPS,
                     "matrices": len(Ws), "elements": numel}
        del g
    del Ws, qs, ws, outs
    torch.cuda.empty_cache()
    return res


def bench_blocksizes(dg, reps=4, rounds=5):
    """The prefill workload with 32, 128 and 256 weights per absmax block, at 64
    without double quantization (fp32 absmax per block), and with the FP4 level table.

    The GEMMs of each variant are timed interleaved with the same GEMM on the plain block-size-64
    weight (``rounds`` alternations of ``reps`` calls) and reported from the medians, with the
    ratio to the plain weight's time: the clock drifts by several percent under these
    power-limited kernels, and the first variant timed after a change of workload ran up to 25%
    slow when each variant was timed once on its own."""
    import synth
    d = torch.device("cuda:0")
    M, K, N = synth.PREFILL_M, synth.PREFILL_K, synth.PREFILL_N
    W = synth.prefill_weight().to(d)
    X = synth.prefill_x().to(d)
    dY = synth.prefill_dy().to(d)
    Y = torch.empty((M, N), dtype=torch.float32, device=d)
    dX = torch.empty((M, K), dtype=torch.float32, device=d)
    Wh = torch.empty((N, K), dtype=torch.bfloat16, device=d)
    flop = 2.0 * M * N * K
    q64 = dg.nf4_quantize(W)
    plain = {"fwd": lambda: dg.nf4_matmul_fwd(X, q64, out=Y), "bwd_dx": lambda: dg.nf4_matmul_bwd_dx(dY, q64, out=dX)}
    out = {}
    for name, bs, dq, qt in (("bs32", 32, True, "nf4"), ("bs128", 128, True, "nf4"), ("bs256", 256, True, "nf4"),
                             ("bs64_no_double_quant", 64, False, "nf4"), ("fp4_bs64", 64, True, "fp4")):
        q = dg.empty_qtensor(N, K, dq, d, bs, qt)
        ws = torch.empty(dg.nf4_sizes(N, K, bs, dq)["workspace_bytes"], dtype=torch.uint8, device=d) if dq else None
        fns = {"quantize": lambda: dg.nf4_quantize(W, blocksize=bs, double_quant=dq, out=q, workspace=ws),
               "fwd": lambda: dg.nf4_matmul_fwd(X, q, out=Y),
               "bwd_dx": lambda: dg.nf4_matmul_bwd_dx(dY, q, out=dX)}
        for fn in fns.values():
            fn()
        torch.cuda.synchronize()
        nb = -(-N * K // bs)
        wq = N * K // 2 + (nb + 4 * (-(-nb // 256)) + 4 if dq else 4 * nb)
        ms = {"quantize": time_events(fns["quantize"], reps)}
        ratio = {}
        for g in ("fwd", "bwd_dx"):
            tv, tp = [], []
            for _ in range(rounds):
                tp.append(time_events(plain[g], reps))
                tv.append(time_events(fns[g], reps))
            ms[g] = float(np.median(tv))
            ratio[g] = ms[g] / float(np.median(tp))
        ms["dequantize"] = time_graph(lambda: dg.nf4_dequantize(q, out=Wh), reps)
        out[name] = {
            "quantize_GB/s": (N * K * 2 + wq) / (ms["quantize"] * 1e-3) / 1e9,
            "dequantize_GB/s": (wq + N * K * 2) / (ms["dequantize"] * 1e-3) / 1e9,
            "fwd_TFLOP/s": flop / (ms["fwd"] * 1e-3) / 1e12,
            "bwd_dx_TFLOP/s": flop / (ms["bwd_dx"] * 1e-3) / 1e12,
            "fwd_time_vs_bs64": ratio["fwd"],
            "bwd_dx_time_vs_bs64": ratio["bwd_dx"],
            "bits_per_weight": 8.0 * wq / (N * K)}
    del W, X, dY, Y, dX, Wh, q64
    torch.cuda.empty_cache()
    return {"blocksize_variants": out}


def bench_tiny(dg, reps=10):
    """The tiny workload (W 256x256 fp32, X and dY 8x256): per-call latency of every call,
    replayed from HIP graphs of 20 calls (latency-bound; reported, not a roofline figure)."""
    import synth
    d = torch.device("cuda:0")
    t = synth.tiny()
    W, X, dY = t["W"].to(d), t["X"].to(d), t["dY"].to(d)
    N, K = W.shape
    out = {}
    for dq in (True, False):
        q = dg.empty_qtensor(N, K, dq, d)
        ws = torch.empty(dg.nf4_sizes(N, K, 64, dq)["workspace_bytes"], dtype=torch.uint8, device=d) if dq else None
        tag = "" if dq else "_no_double_quant"
        out["quantize" + tag] = time_graph(lambda: dg.nf4_quantize(W, double_quant=dq, out=q, workspace=ws), reps) * 1e3
        if dq:
            Wh = torch.empty((N, K), dtype=torch.bfloat16, device=d)
            Y = torch.empty((X.shape[0], N), dtype=torch.float32, device=d)
            dX = torch.empty((dY.shape[0], K), dtype=torch.float32, device=d)
            out["dequantize"] = time_graph(lambda: dg.nf4_dequantize(q, out=Wh), reps) * 1e3
            out["fwd"] = time_graph(lambda: dg.nf4_matmul_fwd(X, q, out=Y), reps) * 1e3
            out["bwd_dx"] = time_graph(lambda: dg.nf4_matmul_bwd_dx(dY, q, out=dX), reps) * 1e3
    return {"tiny_us_per_call": out}


def bench_read_stream(reps=5, gib=4):
    """The achievable HBM read bandwidth: a plain read stream (libnf4_bench) over a 4 GiB buffer
    (16x the 256 MB last-level cache), best of a few launch shapes."""
    import ctypes
    from dequant_gemm_amd.build import BENCH_LIB
    if not os.path.exists(BENCH_LIB):
        raise RuntimeError(f"{BENCH_LIB} is missing: build with `python -m dequant_gemm_amd.build`")
    L = ctypes.CDLL(BENCH_LIB)
    L.nf4bench_read_stream.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int,
                                       ctypes.c_int, ctypes.c_void_p]
    L.nf4bench_read_stream.restype = ctypes.c_int
    d = torch.device("cuda:0")
    nbytes = gib << 30
    src = torch.empty(nbytes, dtype=torch.uint8, device=d)
    shapes = ((1024, 256), (2048, 256), (4096, 256), (1024, 512), (2048, 512), (1024, 1024))
    sink = torch.empty(max(g * b for g, b in shapes), dtype=torch.int32, device=d)
    stream = torch.cuda.current_stream(d).cuda_stream
    best = None
    for grid, block in shapes:
        assert grid * block <= sink.numel()
        call = lambda: L.nf4bench_read_stream(src.data_ptr(), nbytes, sink.data_ptr(), grid, block, stream)
        if call() != 0:
            raise RuntimeError("nf4bench_read_stream failed")
        torch.cuda.synchronize()
        ms = time_events(call, reps)
        gbps = nbytes / (ms * 1e-3) / 1e9
        if best is None or gbps > best["GB/s"]:
            best = {"GB/s": gbps, "frac_hbm": gbps / PEAK_HBM_GBPS, "grid": grid, "block": block,
                    "bytes": nbytes, "what": "plain 16-byte-load read stream, best launch shape"}
    del src, sink
    torch.cuda.empty_cache()
    return {"hbm_read_stream": best}


DECODE_TRACE_KERNELS = ("fwd_small_kernel",)   # the small-M forward's kernel names
DECODE_TRACE_POOL, DECODE_TRACE_ROUNDS = 64, 4


def decode_kernel_trace(timeout_s=300):
    """Decode kernel durations from the profiler: a child process runs the decode calls
    (M = 1, 4, 16 over a pool of 64 quantized 4096x4096 weights, eager launches) under
    `rocprofv3 --kernel-trace`; each dispatch's begin-to-end time excludes launch gaps.
    Runs before this process touches the GPU."""
    import csv
    import glob
    import shutil
    import subprocess
    import tempfile
    prof = shutil.which("rocprofv3")
    if prof is None:
        return {"decode_kernel_trace": None, "decode_kernel_trace_error": "rocprofv3 not found"}
    out = tempfile.mkdtemp(prefix="nf4_decode_trace_")
    cmd = [prof, "--kernel-trace", "--output-format", "csv", "-d", out, "-o", "decode", "--",
           sys.executable, os.path.abspath(__file__), "--op", "decode_trace"]
    try:
        r = subprocess.run(cmd, capture_output=True, text=True, timeout=timeout_s, cwd="/tmp",
                           env=dict(os.environ, TMPDIR="/tmp"))
        files = glob.glob(os.path.join(out, "**", "*kernel_trace.csv"), recursive=True)
        if not files:
            return {"decode_kernel_trace": None,
                    "decode_kernel_trace_error": f"no trace (rc {r.returncode}): {r.stderr[-300:]}"}
        rows = [x for x in csv.DictReader(open(files[0]))
                if any(k in x["Kernel_Name"] for k in DECODE_TRACE_KERNELS)]
        rows.sort(key=lambda x: int(x["Start_Timestamp"]))
        per_m = DECODE_TRACE_POOL * DECODE_TRACE_ROUNDS
        import synth
        if len(rows) != per_m * len(synth.DECODE_MS):
            return {"decode_kernel_trace": None,
                    "decode_kernel_trace_error": f"expected {per_m * len(synth.DECODE_MS)} dispatches, got {len(rows)}"}
        res = {}
        K, N = synth.DECODE_K, synth.DECODE_N
        for i, M in enumerate(synth.DECODE_MS):
            # the first round over the pool is a warm-up
            d = [(int(x["End_Timestamp"]) - int(x["Start_Timestamp"])) * 1e-3
                 for x in rows[i * per_m + DECODE_TRACE_POOL:(i + 1) * per_m]]
            us = float(np.median(d))
            b = M * K * 2 + wq_bytes(N, K) + M * N * 4
            res[f"decode_m{M}"] = {"kernel_us_median": us, "kernel_us_min": float(np.min(d)),
                                   "GB/s": b / (us * 1e-6) / 1e9, "frac_hbm": b / (us * 1e-6) / 1e9 / PEAK_HBM_GBPS,
                                   "dispatches": len(d)}
        return {"decode_kernel_trace": res}
    except (subprocess.TimeoutExpired, OSError, KeyError, ValueError) as e:
        return {"decode_kernel_trace": None, "decode_kernel_trace_error": repr(e)[:300]}
    finally:
        shutil.rmtree(out, ignore_errors=True)


def cpu_baseline(target_s=12.0):
    """The oracle, as it stands, on a bounded sample of the prefill workload."""
    import oracle as O
    import synth
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        blas_threads = os.cpu_count() or 1
    K, N = synth.PREFILL_K, synth.PREFILL_N
    W = synth.prefill_weight()
    rows_w = 1024                      # quantize 1024 of the 11008 weight rows
    t = time.perf_counter()
    qo = O.quantize(W[:rows_w].float().numpy())
    t_q = time.perf_counter() - t
    wh = O.bf16_bits_to_f32(O.dequantize(qo)).reshape(rows_w, K)
    # fwd and bwd on a slice of rows against that weight slice; scale the row count to the time budget
    X = synth.prefill_x()
    dY = synth.prefill_dy()
    m = 64
    while True:
        t = time.perf_counter()
        O.matmul_fwd(X[:m].float().numpy(), wh)
        O.matmul_bwd_dx(dY[:m, :rows_w].float().numpy(), wh)
        dt = time.perf_counter() - t
        if dt > 2.0 or m >= 4096:
            break
        m *= 2
    reps = max(1, int(target_s / max(dt, 1e-3)))
    t = time.perf_counter()
    for _ in range(reps):
        O.matmul_fwd(X[:m].float().numpy(), wh)
        O.matmul_bwd_dx(dY[:m, :rows_w].float().numpy(), wh)
    t_g = (time.perf_counter() - t) / reps
    flop = 2 * (2.0 * m * rows_w * K)
    # per-weight-element time of the quantizer scaled to the full weight, once per step
    t_q_full = t_q * (N / rows_w)
    t_g_full = t_g * (synth.PREFILL_M / m) * (N / rows_w)
    step_flop = 2 * 2.0 * synth.PREFILL_M * N * K
    return {
        "value": step_flop / (t_q_full + t_g_full) / 1e12,
        "unit": "TFLOP/s",
        "cores": int(blas_threads),
        "kind": "oracle",
        "sample": (f"prefill workload: oracle quantize of {rows_w} of {N} weight rows (1 process), "
                   f"fp64 fwd+bwd of {m} rows x {rows_w} weight rows (numpy BLAS, {blas_threads} threads), "
                   f"{reps} reps; scaled linearly to one full step"),
        "seconds": {"quantize_sample": t_q, "gemm_sample": t_g},
        "cpu": _cpu_model(),
    }


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def run_single_op(dg, op, steps, warmup):
    """One operation of the hot path repeated ``steps`` times (for profiler runs)."""
    import synth
    d = torch.device("cuda:0")
    if op == "copy":
        # a plain device copy of known size: calibrates the traffic counters
        src = torch.empty(1 << 28, dtype=torch.float32, device=d).fill_(1.0)
        dst = torch.empty_like(src)
        fn = lambda i: dst.copy_(src)
    elif op == "decode_trace":
        # the decode calls for the kernel trace: a pool of quantized 4096x4096 weights, M = 1, 4, 16,
        # eager launches, a fixed number of rounds over the pool per M
        import synth as S
        K, N = S.DECODE_K, S.DECODE_N
        qs = [dg.nf4_quantize(_device_normal((N, K), 0.02, 1000 + p, d)) for p in range(DECODE_TRACE_POOL)]
        for M in S.DECODE_MS:
            X = S.decode_x(M).to(d)
            Y = torch.empty((M, N), dtype=torch.float32, device=d)
            torch.cuda.synchronize()
            for _ in range(DECODE_TRACE_ROUNDS):
                for q in qs:
                    dg.nf4_matmul_fwd(X, q, out=Y)
            torch.cuda.synchronize()
        print(json.dumps({"op": op, "calls_per_m": DECODE_TRACE_POOL * DECODE_TRACE_ROUNDS}), flush=True)
        return
    elif op == "decode_large":
        # decode at M = 1, 4, 16 on three rotating quantized 28672 x 8192 weights, ``steps`` calls each
        M0, K, N = synth.LARGE_M, synth.LARGE_K, synth.LARGE_N
        qs = [dg.nf4_quantize(_device_normal((N, K), 0.02, 4100 + p, d)) for p in range(LARGE_DECODE_COPIES)]
        for M in synth.DECODE_MS:
            X = _device_normal((M, K), 1.0, 4001, d)
            Y = torch.empty((M, N), dtype=torch.float32, device=d)
            for i in range(warmup + steps):
                dg.nf4_matmul_fwd(X, qs[i % len(qs)], out=Y)
            torch.cuda.synchronize()
        print(json.dumps({"op": op, "calls_per_m": warmup + steps}), flush=True)
        return
    elif op in ("large_fwd", "large_bwd_dx"):
        # the 8192 x 8192 x 28672 GEMMs on the Student-t weight, inputs drawn on the device as in bench_large
        M, K, N = synth.LARGE_M, synth.LARGE_K, synth.LARGE_N
        torch.manual_seed(4000)
        W = (torch.distributions.StudentT(torch.tensor(4.0, device=d)).sample((N, K)) * 0.02).float().contiguous()
        q = dg.nf4_quantize(W)
        del W
        if op == "large_fwd":
            X = _device_normal((M, K), 1.0, 4001, d)
            Y = torch.empty((M, N), dtype=torch.float32, device=d)
            fn = lambda i: dg.nf4_matmul_fwd(X, q, out=Y)
        else:
            dY = _device_normal((M, N), 0.01, 4002, d)
            dX = torch.empty((M, K), dtype=torch.float32, device=d)
            fn = lambda i: dg.nf4_matmul_bwd_dx(dY, q, out=dX)
    elif op in ("decode", "decode_m1"):
        # decode forward on 16 rotating quantized 4096 x 4096 weights, M = 16 (decode) or 1 (decode_m1)
        K, N = synth.DECODE_K, synth.DECODE_N
        Md = 16 if op == "decode" else 1
        qs = [dg.nf4_quantize(w.to(d)) for w in synth.parallel(synth.decode_weight, range(16))]
        X = synth.decode_x(Md).to(d)
        Y = torch.empty((Md, N), dtype=torch.float32, device=d)
        fn = lambda i: dg.nf4_matmul_fwd(X, qs[i % len(qs)], out=Y)
    elif op == "decode_bwd":
        # the backward dX = dY W^ on 16 rotating quantized 4096 x 4096 weights, M = 16
        K, N = synth.DECODE_K, synth.DECODE_N
        qs = [dg.nf4_quantize(w.to(d)) for w in synth.parallel(synth.decode_weight, range(16))]
        dY = synth.normal((16, N), 1.0, 1216).to(d)
        dX = torch.empty((16, K), dtype=torch.float32, device=d)
        fn = lambda i: dg.nf4_matmul_bwd_dx(dY, qs[i % len(qs)], out=dX)
    else:
        M, K, N = synth.PREFILL_M, synth.PREFILL_K, synth.PREFILL_N
        W = synth.prefill_weight().to(d)
        bs = 32 if op.endswith("_bs32") else 64
        op = op[:-5] if op.endswith("_bs32") else op
        q = dg.nf4_quantize(W, blocksize=bs)
        if op == "fwd":
            X = synth.prefill_x().to(d)
            Y = torch.empty((M, N), dtype=torch.float32, device=d)
            fn = lambda i: dg.nf4_matmul_fwd(X, q, out=Y)
        elif op == "bwd_dx":
            dY = synth.prefill_dy().to(d)
            dX = torch.empty((M, K), dtype=torch.float32, device=d)
            fn = lambda i: dg.nf4_matmul_bwd_dx(dY, q, out=dX)
        elif op == "quantize":
            ws = torch.empty(dg.nf4_sizes(N, K)["workspace_bytes"], dtype=torch.uint8, device=d)
            fn = lambda i: dg.nf4_quantize(W, out=q, workspace=ws)
        elif op == "dequantize":
            Wh = torch.empty((N, K), dtype=torch.bfloat16, device=d)
            fn = lambda i: dg.nf4_dequantize(q, out=Wh)
        elif op == "dense_fwd":
            # hipBLASLt's dense bf16 GEMM of the forward's shape (X [M, K] x W^T), for comparison
            X = synth.prefill_x().to(d)
            Wh = dg.nf4_dequantize(q)
            fn = lambda i: torch.matmul(X, Wh.t())
        elif op == "dense_bwd_dx":
            # hipBLASLt's dense bf16 GEMM of the backward's shape (dY [M, N] x W^ [N, K]), for comparison
            dY = synth.prefill_dy().to(d)
            Wh = dg.nf4_dequantize(q)
            fn = lambda i: torch.matmul(dY, Wh)
        else:
            raise ValueError(op)
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    s = torch.cuda.Event(enable_timing=True)
    e = torch.cuda.Event(enable_timing=True)
    s.record()
    for i in range(steps):
        fn(i)
    e.record()
    e.synchronize()
    print(json.dumps({"op": op, "steps": steps, "ms_per_call": s.elapsed_time(e) / steps}), flush=True)


def _rounded(v):
    if isinstance(v, dict):
        return {k: _rounded(x) for k, x in v.items()}
    return round(v, 4) if isinstance(v, float) else v


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=50,
                    help="untimed steps first; the clock under sustained load settles after ~40 steps")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-large", action="store_true", help="skip the 8192x8192x28672 outlier-heavy shape")
    ap.add_argument("--no-bulk", action="store_true", help="skip the 32-layer quantize/dequantize round trip")
    ap.add_argument("--no-blocksizes", action="store_true", help="skip the block-size 32/128/256 variants")
    ap.add_argument("--no-decode-trace", action="store_true",
                    help="skip the profiler run that takes the decode kernels' own durations")
    ap.add_argument("--op", default=None,
                    choices=["fwd", "bwd_dx", "fwd_bs32", "bwd_dx_bs32", "quantize", "dequantize", "dense_fwd", "dense_bwd_dx", "decode", "decode_bwd",
                             "decode_m1", "decode_large", "decode_trace", "large_fwd", "large_bwd_dx", "copy"],
                    help="run only this operation, --steps times (profiler runs); prints its own JSON line")
    ap.add_argument("--write-traffic", metavar="PMC_DIR", default=None,
                    help="write profiles/traffic.json from FETCH_SIZE/WRITE_SIZE counter runs in PMC_DIR and exit")
    a = ap.parse_args()
    if a.write_traffic:
        print(json.dumps(write_traffic(a.write_traffic), indent=1))
        return
    if a.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the NF4 path here is built and timed on a single "
              "MI355X (no sharding, no collectives); run it with --gpus 1", file=sys.stderr)
        sys.exit(2)
    # the profiler child runs first, while this process has not touched the GPU
    trace = decode_kernel_trace() if not (a.op or a.no_decode or a.no_decode_trace) else None
    if not torch.cuda.is_available():
        print("bench.py needs a HIP device", file=sys.stderr)
        sys.exit(1)
    import dequant_gemm_amd as dg
    dg.lib()
    torch.cuda.synchronize()
    if a.op:
        run_single_op(dg, a.op, a.steps, a.warmup)
        return

    pre = bench_prefill(dg, a.steps, a.warmup)
    ops = pre["ops"]
    if not a.no_decode:
        ops.update(bench_decode(dg))
    if trace is not None:
        ops.update(trace)
    ops.update(bench_read_stream())
    ops.update(bench_tiny(dg))
    if not a.no_large:
        ops.update(bench_large(dg))
    if not a.no_bulk:
        ops.update(bench_bulk(dg))
    if not a.no_blocksizes:
        ops.update(bench_blocksizes(dg))
    dom = "fwd" if ops["fwd"]["ms"] >= ops["bwd_dx"]["ms"] else "bwd_dx"
    ach = ops[dom]["TFLOP/s"]
    line = {
        "metric": METRIC,
        "value": round(pre["tflops_step"], 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(pre["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "prefill: M=4096 (8x512 tokens), K=4096, N=11008, NF4 blocksize 64 "
                               "double-quant; step = quantize + fwd + bwd-dX",
                   "M": 4096, "K": 4096, "N": 11008, "blocksize": 64, "double_quant": True},
        "roofline": {"kernel": "fwd_wide_kernel" if dom == "fwd" else "bwd_dx_wide_kernel",
                     "bound": "mfma", "achieved": round(ach, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(ach / PEAK_BF16_TFLOPS, 4),
                     "traffic": measured_traffic("fwd_wide_kernel" if dom == "fwd" else "bwd_dx_wide_kernel")},
        "ops": {k: _rounded(v) for k, v in ops.items()},
    }
    if not a.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline()
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
