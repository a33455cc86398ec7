"""GPU parity of the grouped GEMMs with packed UE8M0 scales
(dg_grouped_fp8_contiguous_ue8m0_packed, dg_grouped_fp8_masked_ue8m0_packed)
against the oracle's unpack-then-grouped-GEMM, on the same bar as the
fp32-scale grouped calls: every output at small sizes over tile instances,
ragged tails and each layout's degenerate cases (padding rows, empty experts,
two experts in one 256-row tile, masked_m of 0 / 1 / M_max / beyond M_max,
forced K splits starting inside a scale word); sampled outputs at the full
workload sizes in the library's own launch configuration.  On inputs whose
every output is exact in fp32 the packed call gives the oracle's bits and the
fp32-scale call's bits exactly.  The packer fills the bytes past the last K
block with the NaN code, so reading one would show."""
from __future__ import annotations

import os

import numpy as np
import pytest
import torch

import oracle
from harness import inputs, workloads
from tests.parity import SENTINEL_BF16, bf16_bits, bits_to_f64, check_close, dev, say, sentinel_bf16

pytestmark = pytest.mark.gpu

PACK = inputs.pack_ue8m0


@pytest.fixture(scope="module")
def dg():
    import moe_grouped_gemm_x128_amd as m
    return m


@pytest.fixture
def force(request):
    def _set(tile=None, splits=None):
        for k in ("DG_FORCE_TILE", "DG_FORCE_SPLITS"):
            os.environ.pop(k, None)
        if tile is not None:
            os.environ["DG_FORCE_TILE"] = tile
        if splits is not None:
            os.environ["DG_FORCE_SPLITS"] = str(splits)
    yield _set
    for k in ("DG_FORCE_TILE", "DG_FORCE_SPLITS"):
        os.environ.pop(k, None)


def run_contig(dg, x, ids, packed=True):
    out = sentinel_bf16((x.m_total, x.n))
    if packed:
        dg.dg_grouped_fp8_contiguous_ue8m0_packed(dev(x.a), dev(PACK(x.sa)), dev(x.b), dev(PACK(x.sb)), out, dev(ids))
    else:
        dg.dg_grouped_fp8_contiguous(dev(x.a), dev(x.sa), dev(x.b), dev(x.sb), out, dev(ids))
    torch.cuda.synchronize()
    return bf16_bits(out)


def run_masked(dg, x, mm):
    out = sentinel_bf16((x.g, x.m_max, x.n))
    dg.dg_grouped_fp8_masked_ue8m0_packed(dev(x.a), dev(PACK(x.sa)), dev(x.b), dev(PACK(x.sb)), out, dev(mm))
    torch.cuda.synchronize()
    return bf16_bits(out)


def contig_ids(x, kind):
    ids = x.m_indices.copy()
    if kind == "empty_expert":
        ids[256:512] = -1                 # expert 1 gets no rows at all
    elif kind == "two_experts":
        ids[128:256] = 2                  # a 256-row tile whose blocks have different experts
        ids[200:256] = -1
    elif kind == "out_of_range":
        ids[:100] = x.g + 5               # ids past G are skipped
    return ids


@pytest.mark.parametrize("tile", [None, "256x256x2x4", "256x256x1x8", "256x128x2x2", "128x128x2x2", "64x64x1x4"])
@pytest.mark.parametrize("k,kind", [(640, "empty_expert"), (384, "two_experts"), (1152, "out_of_range"),
                                    (128, "ragged")])
def test_contiguous_packed_exact(dg, force, tile, k, kind):
    """Exact-output inputs (small integers, power-of-two scales): the packed
    call's bits are the oracle's and the fp32-scale call's, every row."""
    x = inputs.make_contiguous_exact(4, 256, 300, k, seed=inputs.SEED_BASE + 80 + k)
    ids = contig_ids(x, kind)
    force(tile)
    say(f"contiguous ue8m0 packed exact K={k} {kind} tile={tile}")
    got = run_contig(dg, x, ids)
    ref, exact = oracle.grouped_contiguous_ue8m0_packed(x.a, PACK(x.sa), x.b, PACK(x.sb), ids,
                                                        np.full((x.m_total, x.n), SENTINEL_BF16, np.uint16))
    valid = (ids >= 0) & (ids < x.g)
    xv = exact[valid]
    assert np.array_equal(xv.astype(np.float32).astype(np.float64), xv), "inputs are not exact in fp32"
    assert np.all(got[~valid] == SENTINEL_BF16), "padding rows were written"
    assert np.array_equal(got[valid], ref[valid]), \
        f"{int(np.count_nonzero(got[valid] != ref[valid]))} outputs differ from the oracle"
    assert np.array_equal(got, run_contig(dg, x, ids, packed=False)), "differs from the fp32-scale call"


@pytest.mark.parametrize("tile", [None, "256x256x2x4", "128x128x2x2"])
def test_contiguous_packed_random(dg, force, tile):
    """N(0,1) operands with power-of-two 1x128 / 128x128 scales, K = 1664
    (13 K blocks: the last word holds one)."""
    x = inputs.make_contiguous(3, 384, 260, 1664, seed=inputs.SEED_BASE + 85, pow2=True)
    force(tile)
    say(f"contiguous ue8m0 packed random tile={tile}")
    got = run_contig(dg, x, x.m_indices)
    ref, _ = oracle.grouped_contiguous_ue8m0_packed(x.a, PACK(x.sa), x.b, PACK(x.sb), x.m_indices,
                                                    np.full((x.m_total, x.n), SENTINEL_BF16, np.uint16))
    valid = x.m_indices >= 0
    assert np.all(got[~valid] == SENTINEL_BF16), "padding rows were written"
    check_close(bits_to_f64(got[valid]), bits_to_f64(ref[valid]), "contiguous ue8m0 packed random")
    assert np.array_equal(got, run_contig(dg, x, x.m_indices)), "not deterministic"


@pytest.mark.parametrize("tile,splits", [(None, None), ("256x128x1x4", 3), ("256x64x1x4", 7), ("256x256x2x4", 2),
                                         ("128x128x2x2", None), ("64x64x1x4", 5)])
def test_masked_packed(dg, force, tile, splits):
    """masked_m of 0, 1, M_max, beyond M_max and partial; K = 1280 (10 K
    blocks: splits that start inside a scale word)."""
    mm = np.array([0, 1, 96, 300, 50, 64, 65], np.int32)
    g, m_max, n, k = mm.size, 96, 260, 1280
    x = inputs.make_masked(g, m_max, n, k, seed=inputs.SEED_BASE + 86, masked_m=mm, pow2=True)
    force(tile, splits)
    say(f"masked ue8m0 packed tile={tile} splits={splits}")
    got = run_masked(dg, x, mm)
    ref, _ = oracle.grouped_masked_ue8m0_packed(x.a, PACK(x.sa), x.b, PACK(x.sb), mm,
                                                np.full((g, m_max, n), SENTINEL_BF16, np.uint16))
    rows = np.arange(m_max)[None, :] < np.clip(mm, 0, m_max)[:, None]
    assert np.all(got[~rows] == SENTINEL_BF16), "rows past masked_m were written"
    check_close(bits_to_f64(got[rows]), bits_to_f64(ref[rows]), "masked ue8m0 packed")
    assert np.array_equal(got, run_masked(dg, x, mm)), "not deterministic"


def test_masked_packed_graph_replays(dg):
    """The decode call captured into a HIP graph (no split under capture) and
    replayed with masked_m rewritten on the device between replays."""
    g, m_max, n, k = 4, 256, 384, 2048
    x = inputs.make_masked(g, m_max, n, k, seed=inputs.SEED_BASE + 87, masked_m=[256, 0, 1, 100], pow2=True)
    a, sa, b, sb = dev(x.a), dev(PACK(x.sa)), dev(x.b), dev(PACK(x.sb))
    mm = dev(x.masked_m)
    out = sentinel_bf16((g, m_max, n))
    stream = torch.cuda.Stream()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        dg.dg_grouped_fp8_masked_ue8m0_packed(a, sa, b, sb, out, mm)   # warm-up outside the graph
        stream.synchronize()
        with torch.cuda.graph(graph, stream=stream):
            dg.dg_grouped_fp8_masked_ue8m0_packed(a, sa, b, sb, out, mm)
    for i, vals in enumerate(([256, 0, 1, 100], [3, 300, 0, 129], [64, 65, 255, 2])):
        say(f"masked ue8m0 packed graph replay {i} masked_m={vals}")
        mm.copy_(torch.tensor(vals, dtype=torch.int32))
        out.view(torch.int16).fill_(-1)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = bf16_bits(out)
        ref, _ = oracle.grouped_masked_ue8m0_packed(x.a, PACK(x.sa), x.b, PACK(x.sb), np.array(vals, np.int32),
                                                    np.full((g, m_max, n), SENTINEL_BF16, np.uint16))
        rows = np.arange(m_max)[None, :] < np.clip(np.array(vals), 0, m_max)[:, None]
        assert np.all(got[~rows] == SENTINEL_BF16), f"replay {i}: rows past masked_m were written"
        check_close(bits_to_f64(got[rows]), bits_to_f64(ref[rows]), f"replay {i}")


def test_contiguous_packed_full_size(dg):
    """G=8 x 8192 rows (ragged padding), N=4096, K=7168 with power-of-two
    scales in the library's own launch configuration: sampled outputs."""
    shape = [s for s in workloads.contiguous_sweep() if s["g"] == 8 and s["n"] == 4096][0]
    x = inputs.make_contiguous(shape["g"], shape["rows_per_expert"], shape["n"], shape["k"], shape["seed"], pow2=True)
    say(f"{shape['name']} ue8m0 packed")
    bits = run_contig(dg, x, x.m_indices)
    valid = x.m_indices >= 0
    assert np.all(bits[~valid] == SENTINEL_BF16), "padding rows were written"
    assert not np.any(bits[valid] == SENTINEL_BF16), "valid rows left unwritten"
    rng = np.random.default_rng(5)
    rows = np.flatnonzero(valid)[rng.integers(0, int(valid.sum()), 1536)]
    cols = rng.integers(0, x.n, 1536)
    kb = x.k // 128
    vals, wr = oracle.grouped_contiguous_at(x.a, oracle.unpack_ue8m0(PACK(x.sa), kb), x.b,
                                            oracle.unpack_ue8m0(PACK(x.sb), kb), x.m_indices, rows, cols)
    assert wr.all()
    check_close(bits_to_f64(bits[rows, cols]), bits_to_f64(oracle.round_bf16(vals)), "contiguous ue8m0 full")


@pytest.mark.parametrize("g,n,k", [(16, 4096, 7168), (1, 4096, 7168)])
def test_masked_packed_full_size(dg, g, n, k):
    """The decode shapes (M_max = 256, masked_m ~ U{64..192}) in the library's
    own launch configuration (split K for the single group): sampled outputs."""
    shape = [s for s in workloads.masked_sweep() if s["g"] == g and s["n"] == n and s["k"] == k][0]
    x = inputs.make_masked(g, shape["m_max"], n, k, shape["seed"], pow2=True)
    say(f"{shape['name']} ue8m0 packed masked_m={x.masked_m.tolist()}")
    bits = run_masked(dg, x, x.masked_m)
    rows_ok = np.arange(x.m_max)[None, :] < np.clip(x.masked_m, 0, x.m_max)[:, None]
    assert np.all(bits[~rows_ok] == SENTINEL_BF16), "rows past masked_m were written"
    assert not np.any(bits[rows_ok] == SENTINEL_BF16), "valid rows left unwritten"
    rng = np.random.default_rng(6)
    groups = rng.integers(0, g, 1536)
    rows = (rng.random(1536) * np.clip(x.masked_m[groups], 1, x.m_max)).astype(np.int64)
    cols = rng.integers(0, n, 1536)
    kb = k // 128
    vals, wr = oracle.grouped_masked_at(x.a, oracle.unpack_ue8m0(PACK(x.sa), kb), x.b,
                                        oracle.unpack_ue8m0(PACK(x.sb), kb), x.masked_m, groups, rows, cols)
    assert wr.all()
    check_close(bits_to_f64(bits[groups, rows, cols]), bits_to_f64(oracle.round_bf16(vals)), "masked ue8m0 full")
