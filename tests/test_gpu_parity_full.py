"""GPU parity at the full workload sizes, in the launch configuration the
benchmark times (the library's own tile choice), on sampled outputs the
oracle computes one by one: uniform random positions plus the corners, the
last row and column, and the columns on both sides of every 128-column scale
boundary that the sample touches.  Layout properties are checked on the whole
output: padding rows and rows past masked_m keep their sentinel bits, and
every row that must be written is.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from harness import inputs, workloads
from tests.parity import (SENTINEL_BF16, bf16_bits, bits_to_f64, check_close, dev, say,
                          sentinel_bf16)

pytestmark = pytest.mark.gpu

NSAMPLE = 1536


@pytest.fixture(scope="module")
def dg():
    import moe_grouped_gemm_x128_amd as m
    return m


def _positions(rng, m, n, count=NSAMPLE):
    rows = list(rng.integers(0, m, count))
    cols = list(rng.integers(0, n, count))
    extra = [(0, 0), (m - 1, n - 1), (0, n - 1), (m - 1, 0)]
    for c in (127, 128, 2047, 2048, n - 64, n - 1):
        if 0 <= c < n:
            extra.append((int(rng.integers(0, m)), c))
    rows += [r for r, _ in extra]
    cols += [c for _, c in extra]
    return np.array(rows, np.int64), np.array(cols, np.int64)


@pytest.mark.parametrize("shape", workloads.dense_sweep() + [workloads.DENSE_SMALL], ids=lambda s: s["name"])
def test_dense_full_size(dg, shape):
    m, n, k = shape["m"], shape["n"], shape["k"]
    d = inputs.make_dense(m, n, k, seed=shape["seed"])
    say(f"{shape['name']} (tile {dg.select_config(dg.KIND_DENSE, m, n, k)})")
    c = sentinel_bf16((m, n))
    dg.dg_gemm_fp8_nt(dev(d.a), dev(d.sa), dev(d.b), dev(d.sb), c)
    torch.cuda.synchronize()
    bits = bf16_bits(c)
    assert not np.any(bits == SENTINEL_BF16), "some outputs were not written"
    rows, cols = _positions(np.random.default_rng(1), m, n)
    ref = oracle.round_bf16(oracle.gemm_fp8_nt_at(d.a, d.sa, d.b, d.sb, rows, cols))
    check_close(bits_to_f64(bits[rows, cols]), bits_to_f64(ref), shape["name"])


@pytest.mark.parametrize("shape", workloads.contiguous_sweep(), ids=lambda s: s["name"])
def test_contiguous_full_size(dg, shape):
    x = inputs.make_contiguous(shape["g"], shape["rows_per_expert"], shape["n"], shape["k"], shape["seed"])
    say(f"{shape['name']} (tile {dg.select_config(dg.KIND_CONTIGUOUS, x.m_total, x.n, x.k, x.g)})")
    c = sentinel_bf16((x.m_total, x.n))
    dg.dg_grouped_fp8_contiguous(dev(x.a), dev(x.sa), dev(x.b), dev(x.sb), c, dev(x.m_indices))
    torch.cuda.synchronize()
    bits = bf16_bits(c)
    valid = x.m_indices >= 0
    assert np.all(bits[~valid] == SENTINEL_BF16), "padding rows were written"
    assert not np.any(bits[valid] == SENTINEL_BF16), "valid rows left unwritten"
    rows, cols = _positions(np.random.default_rng(2), x.m_total, x.n)
    keep = valid[rows]
    rows, cols = rows[keep], cols[keep]
    vals, wr = oracle.grouped_contiguous_at(x.a, x.sa, x.b, x.sb, x.m_indices, rows, cols)
    assert wr.all()
    check_close(bits_to_f64(bits[rows, cols]), bits_to_f64(oracle.round_bf16(vals)), shape["name"])


@pytest.mark.parametrize("shape", workloads.masked_sweep(), ids=lambda s: s["name"])
def test_masked_full_size(dg, shape):
    x = inputs.make_masked(shape["g"], shape["m_max"], shape["n"], shape["k"], shape["seed"])
    say(f"{shape['name']} masked_m={x.masked_m.tolist()}")
    c = sentinel_bf16((x.g, x.m_max, x.n))
    dg.dg_grouped_fp8_masked(dev(x.a), dev(x.sa), dev(x.b), dev(x.sb), c, dev(x.masked_m))
    torch.cuda.synchronize()
    bits = bf16_bits(c)
    rows_ok = np.arange(x.m_max)[None, :] < np.clip(x.masked_m, 0, x.m_max)[:, None]
    assert np.all(bits[~rows_ok] == SENTINEL_BF16), "rows past masked_m were written"
    assert not np.any(bits[rows_ok] == SENTINEL_BF16), "valid rows left unwritten"
    rng = np.random.default_rng(3)
    groups = rng.integers(0, x.g, NSAMPLE)
    rows = (rng.random(NSAMPLE) * np.clip(x.masked_m[groups], 1, x.m_max)).astype(np.int64)
    cols = rng.integers(0, x.n, NSAMPLE)
    vals, wr = oracle.grouped_masked_at(x.a, x.sa, x.b, x.sb, x.masked_m, groups, rows, cols)
    assert wr.all()
    check_close(bits_to_f64(bits[groups, rows, cols]), bits_to_f64(oracle.round_bf16(vals)), shape["name"])


@pytest.mark.parametrize("shape", [workloads.WGRAD, workloads.K_GROUPED_WGRAD], ids=lambda s: s["name"])
def test_wgrad_full_size(dg, shape):
    w = inputs.make_wgrad(shape["m"], shape["n"], shape["ks"], shape["seed"])
    g = len(w.ks)
    say(f"{shape['name']}")
    if g == 1:
        d = dev(w.d0[0])
        dg.dg_wgrad_fp8_nt(dev(w.a), dev(w.sa), dev(w.b), dev(w.sb), d)
    else:
        d = dev(w.d0)
        dg.dg_k_grouped_wgrad_fp8_nt(dev(w.a), dev(w.sa), dev(w.b), dev(w.sb), d, w.ks)
    torch.cuda.synchronize()
    got = d.cpu().numpy().reshape(g, w.m, w.n)
    rng = np.random.default_rng(4)
    groups = rng.integers(0, g, NSAMPLE)
    rows, cols = _positions(rng, w.m, w.n, NSAMPLE)
    groups = np.concatenate([groups, rng.integers(0, g, rows.size - NSAMPLE)])
    if g == 1:
        vals = oracle.wgrad_at(w.a, w.sa, w.b, w.sb, w.d0[0], rows, cols)
    else:
        vals = oracle.k_grouped_wgrad_at(w.a, w.sa, w.b, w.sb, w.ks, w.d0, groups, rows, cols)
    ref = oracle.round_f32(vals)
    check_close(got[groups, rows, cols], ref, shape["name"])
    # the accumulated part alone is also inside the bound (D0 does not hide errors)
    base = w.d0[groups, rows, cols].astype(np.float64)
    check_close(got[groups, rows, cols] - base, vals - base, shape["name"] + " (D - D0)")
