"""GPU parity of dg_grouped_fp8_contiguous_swiglu: the contiguous grouped GEMM
with SwiGLU and the 1x128 FP8 re-quantise fused into its epilogue.

Two bars:
  * against the oracle: inputs are built so that every GEMM output is exact in
    fp32 (small integers, power-of-two scales; make_contiguous_exact), so the
    bf16 GEMM output is unique and the oracle's composition -- its contiguous
    GEMM, bf16 rounding, then its SwiGLU + 1x128 quantiser -- fixes every code
    and scale.  The bar is the stand-alone quantiser's (tests/test_gpu_swiglu.py):
    scales within 2^-20 (relative), codes equal away from an e4m3 rounding
    midpoint (2^-18 relative margin), one of the two codes next to one;
  * against the unfused GPU path (dg_grouped_fp8_contiguous into bf16 C, then
    dg_swiglu_quantize_fp8_1x128): identical bits, on random N(0,1)-quantised
    operands too, since the fused epilogue rounds to bf16 and then runs the same
    arithmetic as the stand-alone kernel.
Rows whose expert id is -1 (or not in [0, G)) keep their sentinel bytes.  The
small cases run on both instances of the fused epilogue: the default 2x4-wave
tile and the 1x8-wave one (DG_FORCE_TILE)."""
from __future__ import annotations

import os

import numpy as np
import pytest
import torch

import oracle
from harness import inputs
from tests.parity import SENTINEL_BF16, dev, say

pytestmark = pytest.mark.gpu

MARGIN = 2.0 ** -18
Q_SENTINEL = 0x7F          # an e4m3 NaN code: no output of the quantiser
S_SENTINEL = float("nan")


@pytest.fixture(scope="module")
def dg():
    import moe_grouped_gemm_x128_amd as m
    return m


TILES = [None, "256x256x1x8"]


@pytest.fixture
def force_tile():
    def _set(tile):
        os.environ.pop("DG_FORCE_TILE", None)
        if tile is not None:
            os.environ["DG_FORCE_TILE"] = tile
    yield _set
    os.environ.pop("DG_FORCE_TILE", None)


def run_fused(dg, a, sa, b, sb, ids):
    m_total = a.shape[0]
    i = b.shape[1] // 2
    q = torch.full((m_total, i), Q_SENTINEL, dtype=torch.uint8, device="cuda")
    s = torch.full((m_total, i // 128), S_SENTINEL, dtype=torch.float32, device="cuda")
    dg.dg_grouped_fp8_contiguous_swiglu(a, sa, b, sb, q, s, ids)
    torch.cuda.synchronize()
    return q.cpu().numpy(), s.cpu().numpy()


def run_unfused(dg, a, sa, b, sb, ids):
    m_total = a.shape[0]
    n = b.shape[1]
    c = torch.full((m_total, n), -1, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    dg.dg_grouped_fp8_contiguous(a, sa, b, sb, c, ids)
    q = torch.full((m_total, n // 2), Q_SENTINEL, dtype=torch.uint8, device="cuda")
    s = torch.full((m_total, n // 256), S_SENTINEL, dtype=torch.float32, device="cuda")
    dg.dg_swiglu_quantize_fp8_1x128(c, q, s)
    torch.cuda.synchronize()
    return q.cpu().numpy(), s.cpu().numpy()


def oracle_composition(c, ids):
    """The oracle's GEMM (bf16 bits of every valid row), then its SwiGLU + 1x128
    quantiser on those rows; also checks that the inputs made every output exact."""
    bits, exact = oracle.grouped_contiguous(c.a, c.sa, c.b, c.sb, ids,
                                            np.full((c.m_total, c.n), SENTINEL_BF16, np.uint16))
    valid = (ids >= 0) & (ids < c.g)
    xv = exact[valid]
    assert np.array_equal(xv.astype(np.float32).astype(np.float64), xv), "inputs are not exact in fp32"
    q_ref, s_ref, h = oracle.swiglu_quantize_1x128(np.ascontiguousarray(bits[valid]))
    return valid, q_ref, s_ref, h


def check_oracle(q, s, valid, q_ref, s_ref, h, what):
    q, s = q[valid], s[valid]
    assert np.all(np.abs(s.astype(np.float64) - s_ref) <= 2.0 ** -20 * s_ref), f"{what}: scales"
    y = np.clip(h / np.repeat(s_ref.astype(np.float64), 128, axis=1), -448.0, 448.0)
    lo = oracle.e4m3_encode(np.clip(y * (1 - MARGIN), -448.0, 448.0).astype(np.float32))
    hi = oracle.e4m3_encode(np.clip(y * (1 + MARGIN), -448.0, 448.0).astype(np.float32))
    firm = lo == hi
    assert np.array_equal(q[firm], q_ref[firm]), \
        f"{what}: {int(np.count_nonzero(q[firm] != q_ref[firm]))} codes differ away from a midpoint"
    loose = ~firm
    assert np.all((q[loose] == lo[loose]) | (q[loose] == hi[loose])), f"{what}: code outside the bracket"
    assert loose.mean() < 1e-3, f"{what}: {loose.mean():.2e} of the elements near a midpoint"


def check_untouched(q, s, valid, what):
    assert np.all(q[~valid] == Q_SENTINEL), f"{what}: codes of padding rows were written"
    assert np.all(np.isnan(s[~valid])), f"{what}: scales of padding rows were written"


def layout_ids(c, kind):
    ids = c.m_indices.copy()
    if kind == "empty_expert":
        ids[c.m_total // c.g:2 * c.m_total // c.g] = -1          # expert 1 gets no rows
    elif kind == "out_of_range":
        ids[:128] = c.g + 3                                       # ids past G are skipped
    return ids


@pytest.mark.parametrize("g,rows,i,k,kind", [
    (4, 256, 256, 384, "ragged"),          # ragged padding per expert
    (3, 384, 128, 256, "ragged"),          # experts change inside a 256-row tile
    (4, 256, 384, 512, "empty_expert"),
    (2, 512, 256, 128, "out_of_range"),    # one K block
    (1, 128, 128, 7168, "ragged"),         # long K, a single 128-row block
])
@pytest.mark.parametrize("tile", TILES)
def test_fused_swiglu_against_oracle(dg, force_tile, tile, g, rows, i, k, kind):
    c = inputs.make_contiguous_exact(g, rows, 2 * i, k, seed=inputs.SEED_BASE + 70 + g + k)
    ids = layout_ids(c, kind)
    force_tile(tile)
    say(f"fused swiglu vs oracle G={g} rows={rows} I={i} K={k} {kind} tile={tile}")
    args = (dev(c.a), dev(c.sa), dev(c.b), dev(c.sb), dev(ids))
    q, s = run_fused(dg, *args)
    valid, q_ref, s_ref, h = oracle_composition(c, ids)
    check_untouched(q, s, valid, "fused")
    check_oracle(q, s, valid, q_ref, s_ref, h, f"fused G={g} I={i} K={k} {kind}")
    q2, s2 = run_fused(dg, *args)
    assert np.array_equal(q, q2) and np.array_equal(s, s2, equal_nan=True), "second call differs"


@pytest.mark.parametrize("tile", TILES)
@pytest.mark.parametrize("g,rows,i,k", [(4, 384, 256, 384), (8, 256, 512, 1024)])
def test_fused_swiglu_equals_unfused_path(dg, force_tile, tile, g, rows, i, k):
    """Random N(0,1)-quantised operands: the fused call gives the unfused GPU
    path's bits (GEMM into bf16, then the stand-alone SwiGLU quantiser)."""
    c = inputs.make_contiguous(g, rows, 2 * i, k, seed=inputs.SEED_BASE + 90 + g)
    ids = c.m_indices
    force_tile(tile)
    say(f"fused swiglu vs unfused G={g} rows={rows} I={i} K={k} tile={tile}")
    args = (dev(c.a), dev(c.sa), dev(c.b), dev(c.sb), dev(ids))
    q, s = run_fused(dg, *args)
    qu, su = run_unfused(dg, *args)
    valid = ids >= 0
    check_untouched(q, s, valid, "fused")
    assert np.array_equal(q[valid], qu[valid]), \
        f"{int(np.count_nonzero(q[valid] != qu[valid]))} codes differ from the unfused path"
    assert np.array_equal(s[valid], su[valid]), "scales differ from the unfused path"


def test_fused_swiglu_full_size(dg):
    """The MoE workload's first linear layer at full size (8 experts x 8192
    rows with ragged padding, N = 2I = 4096, K = 7168) with exact-output
    operands: every valid row bit-equal to the unfused GPU path, and 24 sampled
    rows (every column) against the oracle's composition."""
    g, rows, n, k = 8, 8192, 4096, 7168
    c = inputs.make_contiguous_exact(g, rows, n, k, seed=inputs.SEED_BASE + 99)
    ids = c.m_indices
    say(f"fused swiglu full size G={g} rows={rows} N={n} K={k}")
    args = (dev(c.a), dev(c.sa), dev(c.b), dev(c.sb), dev(ids))
    q, s = run_fused(dg, *args)
    qu, su = run_unfused(dg, *args)
    valid = ids >= 0
    check_untouched(q, s, valid, "fused full")
    assert np.array_equal(q[valid], qu[valid]), "codes differ from the unfused path"
    assert np.array_equal(s[valid], su[valid]), "scales differ from the unfused path"
    rng = np.random.default_rng(11)
    rows_s = np.sort(rng.choice(np.flatnonzero(valid), 24, replace=False))
    cols = np.arange(n)
    exact, written = oracle.grouped_contiguous_at(c.a, c.sa, c.b, c.sb, ids, np.repeat(rows_s, n),
                                                  np.tile(cols, rows_s.size))
    assert written.all()
    assert np.array_equal(exact.astype(np.float32).astype(np.float64), exact), "inputs are not exact in fp32"
    bits = oracle.round_bf16(exact).reshape(rows_s.size, n)
    q_ref, s_ref, h = oracle.swiglu_quantize_1x128(bits)
    check_oracle(q[rows_s], s[rows_s], np.ones(rows_s.size, bool), q_ref, s_ref, h, "fused full sampled")
