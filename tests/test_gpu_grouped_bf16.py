"""GPU parity of the grouped BF16 GEMMs (dg_grouped_bf16_contiguous,
dg_grouped_bf16_masked) against the oracle's grouped compositions of its BF16
GEMM, on the bar of the dense BF16 call: every output at small sizes over tile
instances and each layout's degenerate cases (padding rows, an empty expert,
two experts in one 256-row tile, ids past G, masked_m of 0 / 1 / M_max / beyond
M_max, forced K splits of the masked call), and sampled outputs at full
workload sizes in the library's own launch configuration.  Rows that must not
be written keep their sentinel bits; every call is repeated and must be
bit-identical."""
from __future__ import annotations

import os

import numpy as np
import pytest
import torch

import oracle
from harness import inputs
from tests.parity import SENTINEL_BF16, bf16_bits, bits_to_f64, check_close, say, sentinel_bf16

pytestmark = pytest.mark.gpu


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


def bf16_dev(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def run_contig(dg, x, ids, n):
    out = sentinel_bf16((x.a.shape[0], n))
    dg.dg_grouped_bf16_contiguous(bf16_dev(x.a), bf16_dev(x.b), out, torch.from_numpy(ids).cuda())
    torch.cuda.synchronize()
    return bf16_bits(out)


def run_masked(dg, x, mm, n):
    g, m_max, _ = x.a.shape
    out = sentinel_bf16((g, m_max, n))
    dg.dg_grouped_bf16_masked(bf16_dev(x.a), bf16_dev(x.b), out, torch.from_numpy(np.asarray(mm, np.int32)).cuda())
    torch.cuda.synchronize()
    return bf16_bits(out)


def contig_ids(ids, g, kind):
    ids = ids.copy()
    if kind == "empty_expert":
        ids[256:512] = -1
    elif kind == "two_experts":
        ids[128:256] = 2                  # a 256-row tile whose two blocks have different experts
        ids[200:256] = -1
    elif kind == "out_of_range":
        ids[:100] = g + 5
    return ids


@pytest.mark.parametrize("tile", [None, "256x256x2x4", "256x256x1x8", "256x128x2x2", "128x128x2x2", "64x64x1x4"])
@pytest.mark.parametrize("k,kind", [(384, "empty_expert"), (192, "two_experts"), (640, "out_of_range"), (64, "ragged")])
def test_contiguous_bf16(dg, force, tile, k, kind):
    g, rows, n = 4, 256, 300
    x = inputs.make_contiguous_bf16(g, rows, n, k, seed=inputs.SEED_BASE + 100 + k)
    ids = contig_ids(x.ctrl, g, kind)
    force(tile)
    say(f"contiguous bf16 K={k} {kind} tile={tile}")
    got = run_contig(dg, x, ids, n)
    ref, _ = oracle.grouped_contiguous_bf16(x.a, x.b, ids, np.full((g * rows, n), SENTINEL_BF16, np.uint16))
    valid = (ids >= 0) & (ids < g)
    assert np.all(got[~valid] == SENTINEL_BF16), "padding rows were written"
    check_close(bits_to_f64(got[valid]), bits_to_f64(ref[valid]), f"contiguous bf16 {kind} {tile}")
    assert np.array_equal(got, run_contig(dg, x, ids, n)), "not deterministic"


@pytest.mark.parametrize("tile,splits", [(None, None), ("256x128x1x4", 3), ("256x64x1x4", 7), ("256x256x2x4", 2),
                                         ("128x128x2x2", None), ("64x64x1x4", 5)])
def test_masked_bf16(dg, force, tile, splits):
    """masked_m of 0, 1, M_max, beyond M_max and partial; K = 1280 (20 K blocks
    of 64 values)."""
    mm = np.array([0, 1, 96, 300, 50, 64, 65], np.int32)
    g, m_max, n, k = mm.size, 96, 260, 1280
    x = inputs.make_masked_bf16(g, m_max, n, k, seed=inputs.SEED_BASE + 101, masked_m=mm)
    force(tile, splits)
    say(f"masked bf16 tile={tile} splits={splits}")
    got = run_masked(dg, x, mm, n)
    ref, _ = oracle.grouped_masked_bf16(x.a, x.b, mm, np.full((g, m_max, n), SENTINEL_BF16, np.uint16))
    rows = np.arange(m_max)[None, :] < np.clip(mm, 0, m_max)[:, None]
    assert np.all(got[~rows] == SENTINEL_BF16), "rows past masked_m were written"
    check_close(bits_to_f64(got[rows]), bits_to_f64(ref[rows]), f"masked bf16 {tile} {splits}")
    assert np.array_equal(got, run_masked(dg, x, mm, n)), "not deterministic"


def test_contiguous_bf16_full_size(dg):
    """G=4 x 4096 rows (ragged padding), N=4096, K=7168: sampled outputs."""
    g, rows, n, k = 4, 4096, 4096, 7168
    x = inputs.make_contiguous_bf16(g, rows, n, k, seed=inputs.SEED_BASE + 102)
    say(f"contiguous bf16 full G={g} rows={rows} N={n} K={k}")
    got = run_contig(dg, x, x.ctrl, n)
    valid = x.ctrl >= 0
    assert np.all(got[~valid] == SENTINEL_BF16), "padding rows were written"
    assert not np.any(got[valid] == SENTINEL_BF16), "valid rows left unwritten"
    rng = np.random.default_rng(7)
    r = np.flatnonzero(valid)[rng.integers(0, int(valid.sum()), 1536)]
    c = rng.integers(0, n, 1536)
    vals = np.empty(r.size)
    for e in range(g):
        sel = np.flatnonzero(x.ctrl[r] == e)
        vals[sel] = oracle.gemm_bf16_nt_at(x.a, x.b[e], r[sel], c[sel])
    check_close(bits_to_f64(got[r, c]), bits_to_f64(oracle.round_bf16(vals)), "contiguous bf16 full")


def test_masked_bf16_full_size(dg):
    """Decode shape: G=4, M_max=256, masked_m ~ U{64..192}, N=4096, K=7168 (the
    library splits K here): sampled outputs."""
    g, m_max, n, k = 4, 256, 4096, 7168
    mm = np.random.default_rng(8).integers(64, 193, g).astype(np.int32)
    x = inputs.make_masked_bf16(g, m_max, n, k, seed=inputs.SEED_BASE + 103, masked_m=mm)
    say(f"masked bf16 full masked_m={mm.tolist()}")
    got = run_masked(dg, x, mm, n)
    rows_ok = np.arange(m_max)[None, :] < mm[:, None]
    assert np.all(got[~rows_ok] == SENTINEL_BF16), "rows past masked_m were written"
    assert not np.any(got[rows_ok] == SENTINEL_BF16), "valid rows left unwritten"
    rng = np.random.default_rng(9)
    gs = rng.integers(0, g, 1536)
    r = (rng.random(1536) * mm[gs]).astype(np.int64)
    c = rng.integers(0, n, 1536)
    vals = np.empty(gs.size)
    for e in range(g):
        sel = np.flatnonzero(gs == e)
        vals[sel] = oracle.gemm_bf16_nt_at(x.a[e], x.b[e], r[sel], c[sel])
    check_close(bits_to_f64(got[gs, r, c]), bits_to_f64(oracle.round_bf16(vals)), "masked bf16 full")
