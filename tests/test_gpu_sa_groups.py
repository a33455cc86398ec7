"""GPU parity of the contiguous GEMM's grouped row-scale fetch: the two-stage
tiles read a tile's A scales for four K blocks at a time into one of two LDS
group buffers, the next tile's first group landing while the current tile's
last groups are still read.  These cases run several tiles per workgroup
(16384 rows x 2048 columns in 256 x 256 tiles: 512 tiles on at most 256
persistent workgroups) with K-block counts of every residue mod 4 (5, 6, 7 and
9 blocks: last groups of one to three blocks), so each buffer hand-over
between tiles is taken; outputs are sampled against the oracle one by one,
padding rows must keep their sentinel bits and every valid row must be
written.  The packed UE8M0 call and the fused SwiGLU epilogue share the
fetch: the first is checked against the oracle, the second against the
unfused GPU path (GEMM into bf16, then the stand-alone SwiGLU quantiser)."""
from __future__ import annotations

import os

import numpy as np
import pytest
import torch

import oracle
from harness import inputs
from tests.parity import SENTINEL_BF16, bf16_bits, bits_to_f64, check_close, dev, say, sentinel_bf16

pytestmark = pytest.mark.gpu

G, ROWS, N = 4, 4096, 2048
NSAMPLE = 1536


@pytest.fixture(scope="module")
def dg():
    import moe_grouped_gemm_x128_amd as m
    return m


@pytest.fixture
def force_tile():
    def _set(tile):
        os.environ.pop("DG_FORCE_TILE", None)
        if tile is not None:
            os.environ["DG_FORCE_TILE"] = tile
    yield _set
    os.environ.pop("DG_FORCE_TILE", None)


def _sample(x, seed):
    rng = np.random.default_rng(seed)
    valid = np.flatnonzero(x.m_indices >= 0)
    rows = valid[rng.integers(0, valid.size, NSAMPLE)]
    # the last valid row of each expert and the tile-row boundaries
    ends = [int(np.flatnonzero(x.m_indices == e).max()) for e in range(x.g)]
    rows = np.concatenate([rows, ends, valid[:1]]).astype(np.int64)
    cols = rng.integers(0, x.n, rows.size).astype(np.int64)
    cols[-x.g - 1:] = x.n - 1
    return rows, cols


def _check(x, bits, sa, sb, name, seed):
    valid = x.m_indices >= 0
    assert np.all(bits[~valid] == SENTINEL_BF16), f"{name}: padding rows were written"
    assert not np.any(bits[valid] == SENTINEL_BF16), f"{name}: valid rows left unwritten"
    rows, cols = _sample(x, seed)
    vals, wr = oracle.grouped_contiguous_at(x.a, sa, x.b, sb, x.m_indices, rows, cols)
    assert wr.all()
    check_close(bits_to_f64(bits[rows, cols]), bits_to_f64(oracle.round_bf16(vals)), name)


@pytest.mark.parametrize("tile", [None, "256x256x2x4", "256x256x1x8"])
@pytest.mark.parametrize("k", [640, 768, 896, 1152])
def test_contiguous_tiles_per_workgroup(dg, force_tile, tile, k):
    x = inputs.make_contiguous(G, ROWS, N, k, seed=inputs.SEED_BASE + 140 + k // 128)
    force_tile(tile)
    say(f"contiguous sa groups K={k} ({k // 128} blocks) tile={tile}")
    c = sentinel_bf16((x.m_total, x.n))
    dg.dg_grouped_fp8_contiguous(dev(x.a), dev(x.sa), dev(x.b), dev(x.sb), c, dev(x.m_indices))
    torch.cuda.synchronize()
    _check(x, bf16_bits(c), x.sa, x.sb, f"contiguous K={k} {tile}", seed=k)


@pytest.mark.parametrize("k", [640, 1152])
def test_contiguous_ue8m0_packed_tiles_per_workgroup(dg, k):
    x = inputs.make_contiguous(G, ROWS, N, k, seed=inputs.SEED_BASE + 150 + k // 128, pow2=True)
    say(f"contiguous packed UE8M0 sa groups K={k}")
    c = sentinel_bf16((x.m_total, x.n))
    dg.dg_grouped_fp8_contiguous_ue8m0_packed(dev(x.a), dev(inputs.pack_ue8m0(x.sa)), dev(x.b),
                                              dev(inputs.pack_ue8m0(x.sb)), c, dev(x.m_indices))
    torch.cuda.synchronize()
    _check(x, bf16_bits(c), x.sa, x.sb, f"contiguous packed K={k}", seed=k + 1)


@pytest.mark.parametrize("tile", [None, "256x256x1x8"])
@pytest.mark.parametrize("k", [640, 1152])
def test_fused_swiglu_tiles_per_workgroup(dg, force_tile, tile, k):
    x = inputs.make_contiguous(G, ROWS, N, k, seed=inputs.SEED_BASE + 160 + k // 128)
    force_tile(tile)
    say(f"fused swiglu sa groups K={k} tile={tile}")
    ids = dev(x.m_indices)
    a, sa, b, sb = dev(x.a), dev(x.sa), dev(x.b), dev(x.sb)
    i = N // 2
    q = torch.full((x.m_total, i), 0xEE, dtype=torch.uint8, device="cuda")
    s = torch.full((x.m_total, i // 128), float("nan"), dtype=torch.float32, device="cuda")
    dg.dg_grouped_fp8_contiguous_swiglu(a, sa, b, sb, q, s, ids)
    c = sentinel_bf16((x.m_total, N))
    dg.dg_grouped_fp8_contiguous(a, sa, b, sb, c, ids)
    qu = torch.full_like(q, 0xEE)
    su = torch.full_like(s, float("nan"))
    dg.dg_swiglu_quantize_fp8_1x128(c, qu, su)
    torch.cuda.synchronize()
    valid = x.m_indices >= 0
    q, s, qu, su = q.cpu().numpy(), s.cpu().numpy(), qu.cpu().numpy(), su.cpu().numpy()
    assert np.all(q[~valid] == 0xEE) and np.all(np.isnan(s[~valid])), "padding rows were written"
    assert np.array_equal(q[valid], qu[valid]), \
        f"{int(np.count_nonzero(q[valid] != qu[valid]))} codes differ from the unfused path"
    assert np.array_equal(s[valid], su[valid]), "scales differ from the unfused path"
