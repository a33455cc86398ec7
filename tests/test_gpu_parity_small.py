"""GPU parity against the CPU oracle at sizes the oracle finishes in seconds:
every output compared, tiles of every kernel instance, ragged M/N tails,
N not a multiple of 4 (scalar epilogue), and the degenerate cases of each
layout (padding rows, empty experts, masked_m of 0 / M_max / beyond M_max,
empty K groups).  Each call is made twice and must be bit-identical."""
from __future__ import annotations

import os

import numpy as np
import pytest
import torch

import oracle
from harness import inputs
from tests.parity import (SENTINEL_BF16, bf16_bits, bits_to_f64, check_close, dev, say,
                          sentinel_bf16)

pytestmark = pytest.mark.gpu

TILES = [None, "256x128x2x2", "256x256x2x4", "256x224x4x2", "192x256x2x4", "128x128x2x2", "128x64x2x2", "64x128x1x4", "64x64x1x4",
         "64x32x2x2"]


@pytest.fixture(scope="module")
def dg():
    import moe_grouped_gemm_x128_amd as m
    return m


@pytest.fixture
def force_tile(request):
    """Force a tile shape (None: the library's own choice)."""
    def _set(tile):
        os.environ.pop("DG_FORCE_TILE", None)
        if tile is not None:
            os.environ["DG_FORCE_TILE"] = tile
    yield _set
    os.environ.pop("DG_FORCE_TILE", None)


def _dense_run(dg, d):
    c = sentinel_bf16((d.m, d.n))
    dg.dg_gemm_fp8_nt(dev(d.a), dev(d.sa), dev(d.b), dev(d.sb), c)
    torch.cuda.synchronize()
    return bf16_bits(c)


def test_dense_small_workload(dg):
    d = inputs.make_dense(128, 256, 512, seed=inputs.SEED_BASE)
    say("dense 128x256x512")
    got = _dense_run(dg, d)
    ref, _ = oracle.gemm_fp8_nt(d.a, d.sa, d.b, d.sb)
    check_close(bits_to_f64(got), bits_to_f64(ref), "dense 128x256x512")
    assert np.array_equal(got, _dense_run(dg, d)), "not deterministic"


@pytest.mark.parametrize("tile", TILES)
@pytest.mark.parametrize("m,n,k", [(1, 1, 128), (17, 130, 128), (257, 390, 384), (64, 2112, 1024),
                                   (300, 1000, 256), (129, 16, 640)])
def test_dense_ragged(dg, force_tile, m, n, k, tile):
    d = inputs.make_dense(m, n, k, seed=inputs.SEED_BASE + 17 + m + n)
    force_tile(tile)
    say(f"dense {m}x{n}x{k} tile={tile}")
    got = _dense_run(dg, d)
    ref, _ = oracle.gemm_fp8_nt(d.a, d.sa, d.b, d.sb)
    check_close(bits_to_f64(got), bits_to_f64(ref), f"dense {m}x{n}x{k} {tile}")
    assert np.array_equal(got, _dense_run(dg, d)), "not deterministic"


def test_dense_special_values(dg):
    """All-ones operands give exactly K; zero scales give exact zeros."""
    m, n, k = 70, 200, 1024
    a = np.full((m, k), 0x38, np.uint8)
    b = np.full((n, k), 0x38, np.uint8)
    sa = np.ones((m, k // 128), np.float32)
    sb = np.ones((2, k // 128), np.float32)
    d = inputs.Dense(m, n, k, a, sa, b, sb)
    say("dense all-ones")
    got = bits_to_f64(_dense_run(dg, d))
    assert np.all(got == k)
    d.sb = np.zeros_like(sb)
    assert np.all(bits_to_f64(_dense_run(dg, d)) == 0.0)


@pytest.mark.parametrize("tile", [None, "128x128x2x2", "64x64x1x4"])
def test_contiguous_small(dg, force_tile, tile):
    c = inputs.make_contiguous(4, 256, 300, 384, seed=inputs.SEED_BASE + 2, max_pad=127)
    ids = c.m_indices.copy()
    ids[256:512] = -1                 # expert 1 gets no rows at all
    ids[768:768 + 128] = 3            # expert 3: exactly one full 128-row block ...
    ids[768 + 128:] = -1              # ... followed by a whole padding block
    force_tile(tile)
    out = sentinel_bf16((c.m_total, c.n))
    say(f"contiguous G=4 tile={tile}")
    dg.dg_grouped_fp8_contiguous(dev(c.a), dev(c.sa), dev(c.b), dev(c.sb), out, dev(ids))
    torch.cuda.synchronize()
    got = bf16_bits(out)
    ref, _ = oracle.grouped_contiguous(c.a, c.sa, c.b, c.sb, ids,
                                       np.full((c.m_total, c.n), SENTINEL_BF16, np.uint16))
    valid = ids >= 0
    assert np.all(got[~valid] == SENTINEL_BF16), "padding rows were written"
    check_close(bits_to_f64(got[valid]), bits_to_f64(ref[valid]), "contiguous small")


@pytest.mark.parametrize("tile", [None, "256x32x4x1", "256x256x1x8", "256x224x4x2", "256x128x1x4", "256x128x2x2",
                                  "128x128x2x2", "64x32x2x2"])
def test_masked_small(dg, force_tile, tile):
    g, m_max, n, k = 5, 96, 260, 256
    mm = np.array([0, 1, 96, 200, 50], np.int32)  # empty, one row, full, clamped, partial
    x = inputs.make_masked(g, m_max, n, k, seed=inputs.SEED_BASE + 3, masked_m=mm)
    force_tile(tile)
    out = sentinel_bf16((g, m_max, n))
    say(f"masked G=5 tile={tile}")
    dg.dg_grouped_fp8_masked(dev(x.a), dev(x.sa), dev(x.b), dev(x.sb), out, dev(mm))
    torch.cuda.synchronize()
    got = bf16_bits(out)
    ref, _ = oracle.grouped_masked(x.a, x.sa, x.b, x.sb, mm, np.full((g, m_max, n), SENTINEL_BF16, np.uint16))
    rows = np.arange(m_max)[None, :] < np.clip(mm, 0, m_max)[:, None]
    assert np.all(got[~rows] == SENTINEL_BF16), "masked rows were written"
    check_close(bits_to_f64(got[rows]), bits_to_f64(ref[rows]), "masked small")


@pytest.mark.parametrize("tile", [None, "256x224x4x2", "224x256x1x8", "256x128x2x2", "128x128x2x2", "64x128x1x4"])
def test_wgrad_small(dg, force_tile, tile):
    w = inputs.make_wgrad(200, 130, [384], seed=inputs.SEED_BASE + 4)
    force_tile(tile)
    d = dev(w.d0[0])
    say(f"wgrad 200x130x384 tile={tile}")
    dg.dg_wgrad_fp8_nt(dev(w.a), dev(w.sa), dev(w.b), dev(w.sb), d)
    torch.cuda.synchronize()
    ref, _ = oracle.wgrad(w.a, w.sa, w.b, w.sb, w.d0[0])
    check_close(d.cpu().numpy(), ref, "wgrad small")


@pytest.mark.parametrize("m,n,tile", [(130, 72, None), (500, 300, None), (500, 300, "256x256x1x8")])
def test_k_grouped_wgrad_small(dg, force_tile, m, n, tile):
    ks = [128, 0, 256, 384]
    w = inputs.make_wgrad(m, n, ks, seed=inputs.SEED_BASE + 5)
    force_tile(tile)
    d = dev(w.d0)
    say(f"k-grouped wgrad {m}x{n} ks=[128,0,256,384] tile={tile}")
    dg.dg_k_grouped_wgrad_fp8_nt(dev(w.a), dev(w.sa), dev(w.b), dev(w.sb), d, ks)
    torch.cuda.synchronize()
    ref, _ = oracle.k_grouped_wgrad(w.a, w.sa, w.b, w.sb, ks, w.d0)
    got = d.cpu().numpy()
    assert np.array_equal(got[1], w.d0[1]), "empty group's D changed"
    for g in (0, 2, 3):
        check_close(got[g], ref[g], f"k-grouped group {g}")


def test_page_call_style(dg):
    """The pages' call style: (fp8, scale) tuples and a preallocated bf16 output."""
    d = inputs.make_dense(256, 2112, 256, seed=inputs.SEED_BASE + 9)
    lhs = (dev(d.a).view(torch.float8_e4m3fn), dev(d.sa))
    rhs = (dev(d.b).view(torch.float8_e4m3fn), dev(d.sb))
    assert tuple(rhs[1].shape) == (17, 2)
    out = torch.empty(256, 2112, dtype=torch.bfloat16, device="cuda")
    say("page-style dense 256x2112x256")
    dg.gemm_fp8_fp8_bf16_nt(lhs, rhs, out)
    torch.cuda.synchronize()
    ref, _ = oracle.gemm_fp8_nt(d.a, d.sa, d.b, d.sb)
    check_close(bits_to_f64(bf16_bits(out)), bits_to_f64(ref), "page-style dense")


@pytest.mark.parametrize("tile", [None, "256x32x4x1", "256x16x4x1", "256x256x1x8", "256x128x1x4", "256x256x2x4"])
def test_masked_row_quarters(dg, force_tile, tile):
    """Tall masked tiles skip 64-row quarters past masked_m: every boundary."""
    mm = np.array([0, 1, 63, 64, 65, 127, 128, 129, 191, 192, 193, 255, 256, 300], np.int32)
    g, m_max, n, k = mm.size, 256, 136, 256
    x = inputs.make_masked(g, m_max, n, k, seed=inputs.SEED_BASE + 31, masked_m=mm)
    force_tile(tile)
    out = sentinel_bf16((g, m_max, n))
    say(f"masked quarters G={g} tile={tile}")
    dg.dg_grouped_fp8_masked(dev(x.a), dev(x.sa), dev(x.b), dev(x.sb), out, dev(mm))
    torch.cuda.synchronize()
    got = bf16_bits(out)
    ref, _ = oracle.grouped_masked(x.a, x.sa, x.b, x.sb, mm, np.full((g, m_max, n), SENTINEL_BF16, np.uint16))
    rows = np.arange(m_max)[None, :] < np.clip(mm, 0, m_max)[:, None]
    assert np.all(got[~rows] == SENTINEL_BF16), "masked rows were written"
    check_close(bits_to_f64(got[rows]), bits_to_f64(ref[rows]), "masked quarters")


@pytest.fixture
def force_splits():
    def _set(s):
        if s is None:
            os.environ.pop("DG_FORCE_SPLITS", None)
        else:
            os.environ["DG_FORCE_SPLITS"] = str(s)
    yield _set
    os.environ.pop("DG_FORCE_SPLITS", None)


@pytest.mark.parametrize("tile", ["64x32x2x2", "128x128x2x2", "256x256x1x8", "256x224x4x2", "192x256x2x4"])
@pytest.mark.parametrize("splits", [2, 3, 4, 10])
@pytest.mark.parametrize("m,n,k", [(70, 300, 1280), (1, 130, 512), (200, 2112, 1792)])
def test_dense_split_k(dg, force_tile, force_splits, m, n, k, tile, splits):
    """K split over workgroups, partials summed by the reduction kernel; K
    blocks not divisible by the split count (uneven last chunk)."""
    d = inputs.make_dense(m, n, k, seed=inputs.SEED_BASE + 41 + m + k)
    force_tile(tile)
    force_splits(splits)
    say(f"dense split-K {m}x{n}x{k} tile={tile} splits={splits}")
    got = _dense_run(dg, d)
    ref, _ = oracle.gemm_fp8_nt(d.a, d.sa, d.b, d.sb)
    check_close(bits_to_f64(got), bits_to_f64(ref), f"dense split {m}x{n}x{k} {tile} s{splits}")
    assert np.array_equal(got, _dense_run(dg, d)), "split-K result not deterministic"


@pytest.mark.parametrize("tile", ["256x32x4x1", "256x256x1x8", "256x64x1x4", "64x32x2x2"])
@pytest.mark.parametrize("splits", [2, 5])
def test_masked_split_k(dg, force_tile, force_splits, tile, splits):
    mm = np.array([0, 1, 96, 300, 50, 64, 65], np.int32)  # empty, one row, full, clamped, partial
    g, m_max, n, k = mm.size, 96, 260, 1280
    x = inputs.make_masked(g, m_max, n, k, seed=inputs.SEED_BASE + 43, masked_m=mm)
    force_tile(tile)
    force_splits(splits)
    say(f"masked split-K G={g} tile={tile} splits={splits}")

    def run():
        out = sentinel_bf16((g, m_max, n))
        dg.dg_grouped_fp8_masked(dev(x.a), dev(x.sa), dev(x.b), dev(x.sb), out, dev(mm))
        torch.cuda.synchronize()
        return bf16_bits(out)
    got = run()
    ref, _ = oracle.grouped_masked(x.a, x.sa, x.b, x.sb, mm, np.full((g, m_max, n), SENTINEL_BF16, np.uint16))
    rows = np.arange(m_max)[None, :] < np.clip(mm, 0, m_max)[:, None]
    assert np.all(got[~rows] == SENTINEL_BF16), "masked rows were written"
    check_close(bits_to_f64(got[rows]), bits_to_f64(ref[rows]), f"masked split {tile} s{splits}")
    assert np.array_equal(got, run()), "split-K result not deterministic"


def test_split_k_under_graph_capture(dg):
    """A call captured into a HIP graph does not split (no allocation while
    capturing); its replays match the eager split-K result."""
    d = inputs.make_dense(64, 2112, 7168, seed=inputs.SEED_BASE + 47)
    assert dg.select_config(dg.KIND_DENSE, 64, 2112, 7168)["k_splits"] > 1
    say("dense 64x2112x7168 eager (split) vs graph (no split)")
    a, sa, b, sb = dev(d.a), dev(d.sa), dev(d.b), dev(d.sb)
    eager = sentinel_bf16((d.m, d.n))
    dg.dg_gemm_fp8_nt(a, sa, b, sb, eager)
    torch.cuda.synchronize()
    out = sentinel_bf16((d.m, d.n))
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        dg.dg_gemm_fp8_nt(a, sa, b, sb, out)  # warm up on the side stream
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=s):
            dg.dg_gemm_fp8_nt(a, sa, b, sb, out)
    ref, _ = oracle.gemm_fp8_nt(d.a, d.sa, d.b, d.sb)
    e = bf16_bits(eager)
    check_close(bits_to_f64(e), bits_to_f64(ref), "eager split")
    for rep in range(3):
        out.fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        check_close(bits_to_f64(bf16_bits(out)), bits_to_f64(ref), f"graph replay {rep}")


@pytest.mark.parametrize("tile", [None, "256x256x2x4", "256x256x1x8", "256x128x2x2", "128x128x2x2"])
def test_contiguous_tall_tiles(dg, force_tile, tile):
    """256-row tiles span two 128-row blocks: a pair with one expert, a pair
    whose blocks belong to different experts (computed in two passes), a
    padding block next to an expert, a partial block, and a last tile of only
    128 rows (M_total not a multiple of 256)."""
    c = inputs.make_contiguous(4, 384, 270, 384, seed=inputs.SEED_BASE + 53, max_pad=0)
    m_total = 9 * 128
    blocks = [0, 0, 0, 1, -1, 2, 2, 3, 1]          # expert of each 128-row block
    valid = [128, 128, 100, 128, 0, 128, 128, 50, 77]  # valid rows at the start of each block
    ids = np.full(m_total, -1, np.int32)
    for i, (e, v) in enumerate(zip(blocks, valid)):
        ids[i * 128:i * 128 + v] = e
    a, sa = np.ascontiguousarray(c.a[:m_total]), np.ascontiguousarray(c.sa[:m_total])
    force_tile(tile)
    out = sentinel_bf16((m_total, c.n))
    say(f"contiguous tall tiles tile={tile}")
    dg.dg_grouped_fp8_contiguous(dev(a), dev(sa), dev(c.b), dev(c.sb), out, dev(ids))
    torch.cuda.synchronize()
    got = bf16_bits(out)
    ref, _ = oracle.grouped_contiguous(a, sa, c.b, c.sb, ids, np.full((m_total, c.n), SENTINEL_BF16, np.uint16))
    ok = ids >= 0
    assert np.all(got[~ok] == SENTINEL_BF16), "padding rows were written"
    assert not np.any(got[ok] == SENTINEL_BF16), "valid rows left unwritten"
    check_close(bits_to_f64(got[ok]), bits_to_f64(ref[ok]), f"contiguous tall {tile}")


@pytest.mark.parametrize("tile", ["256x32x4x1", None])
@pytest.mark.parametrize("splits", [None, 2, 3])
@pytest.mark.parametrize("k", [512, 2048])
def test_masked_decode_kernels(dg, force_tile, force_splits, tile, splits, k):
    """The masked decode tiles at longer K: ragged N (a last column tile
    narrower than the tile), every row-quarter boundary of masked_m, forced K
    splits (an uneven last split)."""
    mm = np.array([0, 1, 63, 64, 65, 128, 191, 192, 255, 256, 300], np.int32)
    g, m_max, n = mm.size, 256, 392
    x = inputs.make_masked(g, m_max, n, k, seed=inputs.SEED_BASE + 61 + k, masked_m=mm)
    force_tile(tile)
    force_splits(splits)
    say(f"masked decode kernel={tile} K={k} splits={splits}")

    def run():
        out = sentinel_bf16((g, m_max, n))
        dg.dg_grouped_fp8_masked(dev(x.a), dev(x.sa), dev(x.b), dev(x.sb), out, dev(mm))
        torch.cuda.synchronize()
        return bf16_bits(out)
    got = run()
    ref, _ = oracle.grouped_masked(x.a, x.sa, x.b, x.sb, mm, np.full((g, m_max, n), SENTINEL_BF16, np.uint16))
    rows = np.arange(m_max)[None, :] < np.clip(mm, 0, m_max)[:, None]
    assert np.all(got[~rows] == SENTINEL_BF16), "masked rows were written"
    assert not np.any(got[rows] == SENTINEL_BF16), "valid rows left unwritten"
    check_close(bits_to_f64(got[rows]), bits_to_f64(ref[rows]), f"masked decode {tile} K={k} s{splits}")
    assert np.array_equal(got, run()), "not deterministic"
