"""GPU: the library's calls captured in a HIP graph and replayed.

The benchmark replays decode, dequantize and bulk passes from HIP graphs, so
every call must be capturable (no host synchronisation, no memset node) and
give the eager result on every replay.  Between replays the program does
eager work of its own (a different quantization into other buffers, torch
kernels) and synchronises, and each replay is checked bit for bit against
the eager results of the same calls.
"""
import numpy as np
import pytest
import torch

import synth
from tests._gpu import bf16_bits, dev, lib

pytestmark = pytest.mark.gpu


def test_graph_replays_match_eager():
    dg = lib()
    d = dev()
    N, K = 1536, 1024
    W = synth.normal((N, K), 0.02, 700, torch.bfloat16).to(d)
    X1 = synth.normal((4, K), 1.0, 701).to(d)           # small-M kernel
    X2 = synth.normal((300, K), 1.0, 702).to(d)         # large-M kernel
    dY = synth.normal((300, N), 1.0, 703).to(d)
    U = synth.normal((300, 32), 1.0, 704).to(d)
    B = synth.normal((N, 32), 0.1, 705).to(d)
    q = dg.empty_qtensor(N, K, True, d)
    ws = torch.empty(dg.nf4_sizes(N, K)["workspace_bytes"], dtype=torch.uint8, device=d)
    Wh = torch.empty((N, K), dtype=torch.bfloat16, device=d)
    Y1 = torch.empty((4, N), device=d)
    Y2 = torch.empty((300, N), device=d)
    Y3 = torch.empty((300, N), device=d)
    dX = torch.empty((300, K), device=d)

    def calls():
        dg.nf4_quantize(W, out=q, workspace=ws)
        dg.nf4_dequantize(q, out=Wh)
        dg.nf4_matmul_fwd(X1, q, out=Y1)
        dg.nf4_matmul_fwd(X2, q, out=Y2)
        dg.nf4_matmul_bwd_dx(dY, q, out=dX)
        dg.nf4_matmul_fwd_lora(X2, q, U, B, out=Y3)

    calls()
    torch.cuda.synchronize()
    want = [t.clone() for t in (q.packed, q.absmax_q, q.absmax_scale, q.absmax_mean, Wh, Y1, Y2, dX, Y3)]
    outs = (q.packed, q.absmax_q, q.absmax_scale, q.absmax_mean, Wh, Y1, Y2, dX, Y3)

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        calls()
    W2 = synth.normal((N, K), 0.05, 706, torch.bfloat16).to(d)
    for rep in range(4):
        for t in outs:
            t.zero_()                                   # clear every output before the replay
        # eager work between replays: another quantization into other buffers, torch kernels
        q2 = dg.nf4_quantize(W2)
        _ = dg.nf4_matmul_fwd(X2, q2)
        _ = (X2.float() @ X2.float().t()).sum()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (got, exp) in enumerate(zip(outs, want)):
            assert torch.equal(got.view(torch.uint8), exp.view(torch.uint8)), f"replay {rep}, output {i}"
