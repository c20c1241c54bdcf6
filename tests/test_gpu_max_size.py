"""Parity at the largest tensor the library accepts: 2^36 elements.

The library limits a quantized tensor to 2^36 elements; at block size 32 that is
2^31 blocks, the most any call handles (block counts, the exact-mean digit sums
and the division of the mean are at their widest there).  The weight is
2^20 x 2^16 bf16 (128 GiB), built on the device from one seeded 64 x 65536 tile:
tile t (64 rows) is the base tile times 2^k_t, k_t from a fixed set of
exponents.  Scaling by a power of two is exact and leaves every quotient x / a
unchanged, so each block's absmax is the base block's times 2^k_t and its codes
are the base block's codes.  The oracle therefore quantizes the base tile once;
the mean of all 2^31 absmax values is the exact rational S_base * sum_t 2^k_t /
2^31 (S_base: the exact sum over the base tile), rounded by the oracle's
rational-to-fp32 routine; a tile's 512 groups of 256 blocks never straddle
tiles, so its int8 absmax, scales and W^ are the oracle's double quantization
and dequantization of the scaled base tile under that mean.  The CPU test below
checks this decomposition against the oracle run on a whole (small) tiled
weight.  On the GPU every code, int8 absmax, scale and W^ element is compared,
tile by tile on the device against the oracle's per-exponent expectations; the
fused GEMMs at this size on sampled outputs.
"""
import numpy as np
import pytest
import torch

import oracle as O
import synth
from tests._gpu import assert_gemm_within_bound, dev, lib, note, u32

BS = 32
TILE_ROWS = 64
EXPS = (-6, -2, 0, 1, 3, 5)


def tile_exponents(ntiles: int) -> np.ndarray:
    return np.asarray(EXPS)[(7 * np.arange(ntiles)) % len(EXPS)]


def exact_units_sum(a: np.ndarray) -> int:
    """Sum of float32 values as an exact integer count of 2^-149 units."""
    return sum(int(v) for v in (np.asarray(a, np.float32).astype(np.float64) * 2.0 ** 149).tolist())


def class_expectations(base: np.ndarray, exps: np.ndarray, bs: int = BS) -> dict:
    """Oracle results for a weight whose tile t is ``base`` * 2^exps[t].

    Returns the base tile's packed codes, the mean of all block absmax values,
    and per exponent k the int8 absmax, group scales and W^ bits of one tile.
    """
    base = np.asarray(base, np.float32)
    a0 = O.block_absmax(base.ravel(), bs)
    assert (a0.size % O.DQ_GROUP) == 0, "a tile must hold whole groups"
    codes = O.encode_blocks(base.reshape(-1, bs), a0).ravel()
    kmin = int(exps.min())
    e_sum = sum(1 << (int(k) - kmin) for k in exps)              # sum_t 2^(k_t - kmin)
    num = exact_units_sum(a0) * e_sum
    den = (a0.size * exps.size) << 149
    mu = O.round_rational_to_f32(num << kmin, den) if kmin >= 0 else O.round_rational_to_f32(num, den << -kmin)
    per = {}
    for k in sorted(set(int(k) for k in exps)):
        ak = np.ldexp(a0, k).astype(np.float32)                   # exact
        q, s = O.double_quant(ak, mu)
        per[k] = {"q": q, "s": s, "what": O.dequantize_codes(codes, O.dq_absmax(q, s, mu), bs)}
    return {"packed": O.pack_codes(codes), "mean": mu, "per": per}


def test_tiled_decomposition_matches_the_whole_oracle():
    """The per-tile expectations equal the oracle run on the whole tiled weight (CPU)."""
    base = synth.normal((8, 1024), 0.02, 5100, torch.bfloat16).float().numpy()   # 256 blocks of 32
    exps = tile_exponents(11)
    w = np.concatenate([np.ldexp(base, int(k)).astype(np.float32) for k in exps])
    whole = O.quantize(w, blocksize=BS, double_quant_on=True)
    want = class_expectations(base, exps)
    assert np.float32(whole["mean"]).view(np.uint32) == np.float32(want["mean"]).view(np.uint32)
    nb = base.size // BS
    wh = O.dequantize(whole)
    for t, k in enumerate(exps):
        per = want["per"][int(k)]
        assert np.array_equal(whole["packed"][t * base.size // 2:(t + 1) * base.size // 2], want["packed"])
        assert np.array_equal(whole["absmax_q"][t * nb:(t + 1) * nb], per["q"])
        assert np.array_equal(whole["scale"][t * nb // 256:(t + 1) * nb // 256].view(np.uint32), per["s"].view(np.uint32))
        assert np.array_equal(wh[t * base.size:(t + 1) * base.size], per["what"])


@pytest.fixture(scope="module")
def max_weight():
    dg = lib()
    d = dev()
    rows, cols = 1 << 20, 1 << 16
    assert rows * cols == 1 << 36
    ntiles = rows // TILE_ROWS
    base_bf16 = synth.normal((TILE_ROWS, cols), 0.02, 5000, torch.bfloat16)
    exps = tile_exponents(ntiles)
    note("max size: oracle on the base tile")
    want = class_expectations(base_bf16.float().numpy(), exps)
    note(f"max size: building the {rows}x{cols} bf16 weight on the device")
    W = torch.empty((rows, cols), dtype=torch.bfloat16, device=d)
    Wv = W.view(ntiles, TILE_ROWS, cols)
    b = base_bf16.to(d).float()
    for k in want["per"]:
        idx = torch.from_numpy(np.nonzero(exps == k)[0]).to(d)
        Wv[idx] = (b * 2.0 ** k).to(torch.bfloat16)               # exact power-of-two scaling
    note(f"max size: quantize ({rows * cols} elements, block size {BS})")
    q = dg.nf4_quantize(W, blocksize=BS, double_quant=True)
    torch.cuda.synchronize()
    assert q.packed.numel() == 1 << 35 and q.absmax_q.numel() == 1 << 31 and q.absmax_scale.numel() == 1 << 23
    del W, Wv
    yield dg, q, want, exps, (rows, cols)
    del q
    torch.cuda.empty_cache()


def _tiles_equal(dev_view: torch.Tensor, tiles: np.ndarray, want: torch.Tensor, what: str, chunk: int = 256):
    """dev_view[t] == want for every t in ``tiles``, compared on the device in chunks."""
    d = dev_view.device
    for lo in range(0, tiles.size, chunk):
        idx = torch.from_numpy(tiles[lo:lo + chunk]).to(d)
        eq = dev_view[idx] == want
        if not bool(eq.all()):
            bad = (~eq).nonzero()[0].tolist()
            pytest.fail(f"max size {what}: tile {int(tiles[lo + bad[0]])}, offset {bad[1:]} differs")


@pytest.mark.gpu
def test_state_codes_and_dequantized_weight(max_weight):
    dg, q, want, exps, (rows, cols) = max_weight
    d = dev()
    ntiles = exps.size
    assert u32(q.absmax_mean)[0] == np.float32(want["mean"]).view(np.uint32)
    note("max size: codes of every tile")
    alltiles = np.arange(ntiles)
    _tiles_equal(q.packed.view(ntiles, -1), alltiles, torch.from_numpy(want["packed"]).to(d), "packed")
    qv = q.absmax_q.view(ntiles, -1)
    sv = q.absmax_scale.view(torch.int32).view(ntiles, -1)
    for k, per in want["per"].items():
        tiles = np.nonzero(exps == k)[0]
        note(f"max size: int8 absmax and scales, 2^{k} tiles ({tiles.size})")
        _tiles_equal(qv, tiles, torch.from_numpy(per["q"]).to(d), f"int8 absmax (2^{k})")
        _tiles_equal(sv, tiles, torch.from_numpy(per["s"].view(np.int32)).to(d), f"scales (2^{k})")
    note("max size: dequantize")
    wh = dg.nf4_dequantize(q, torch.bfloat16)
    torch.cuda.synchronize()
    whv = wh.view(torch.int16).view(ntiles, -1)
    for k, per in want["per"].items():
        tiles = np.nonzero(exps == k)[0]
        note(f"max size: W^ of the 2^{k} tiles")
        _tiles_equal(whv, tiles, torch.from_numpy(per["what"].view(np.int16)).to(d), f"W^ (2^{k})", chunk=128)
    del wh, whv
    torch.cuda.empty_cache()


def _what_rows(want, exps, ns, cols):
    """W^ rows ns (float32) from the per-exponent tile expectations."""
    out = np.empty((ns.size, cols), np.float32)
    for i, n in enumerate(ns):
        w = want["per"][int(exps[n // TILE_ROWS])]["what"].reshape(TILE_ROWS, cols)
        out[i] = O.bf16_bits_to_f32(w[n % TILE_ROWS])
    return out


@pytest.mark.gpu
@pytest.mark.parametrize("M", [4, 32])
def test_forward_at_max_size(max_weight, M):
    dg, q, want, exps, (rows, cols) = max_weight
    d = dev()
    note(f"max size: forward M={M}")
    X = synth.normal((M, cols), 1.0, 5010 + M)
    Y = dg.nf4_matmul_fwd(X.to(d), q)
    torch.cuda.synchronize()
    rng = np.random.default_rng(5020 + M)
    ns = np.unique(np.concatenate([rng.integers(0, rows, 384), np.arange(64), np.arange(rows - 64, rows)]))
    wr = _what_rows(want, exps, ns, cols)
    x = X.float().numpy()
    assert_gemm_within_bound(Y[:, torch.from_numpy(ns).to(d)], O.matmul_fwd(x, wr), O.fwd_bound(x, wr),
                             f"max size fwd M={M}")


@pytest.mark.gpu
def test_backward_at_max_size(max_weight):
    dg, q, want, exps, (rows, cols) = max_weight
    d = dev()
    M = 4
    note("max size: backward dX, M=4 (reduction over 2^20 rows)")
    dY = synth.normal((M, rows), 1.0, 5030)
    dX = dg.nf4_matmul_bwd_dx(dY.to(d), q)
    torch.cuda.synchronize()
    rng = np.random.default_rng(5031)
    ks = np.unique(np.concatenate([rng.integers(0, cols, 96), np.arange(16), np.arange(cols - 16, cols)]))
    # W^[:, ks] for every row: tile t takes its exponent class's tile
    klist = sorted(want["per"])
    cls = np.searchsorted(klist, exps)
    tiles = np.stack([O.bf16_bits_to_f32(want["per"][k]["what"]).reshape(TILE_ROWS, cols)[:, ks] for k in klist])
    wc = tiles[cls].reshape(rows, ks.size)
    dy = dY.float().numpy()
    assert_gemm_within_bound(dX[:, torch.from_numpy(ks).to(d)], O.matmul_bwd_dx(dy, wc), O.bwd_dx_bound(dy, wc),
                             "max size bwd")
