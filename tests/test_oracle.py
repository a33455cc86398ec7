"""Pins for the CPU oracle (no GPU).  Each test checks the oracle against
something other than itself: torch's own e4m3 decode and bf16 cast, numpy's
fp32 cast and fp64 matmul, an exact integer/rational brute force
(tests/exact_ref.py), closed forms, and invariants of the grouped layouts.
"""
from __future__ import annotations

import hashlib
import json
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from harness import inputs
from tests import exact_ref as X

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rand_codes(rng, shape, nan_free=True):
    c = rng.integers(0, 256, size=shape, dtype=np.uint8)
    if nan_free:
        c[(c & 0x7F) == 0x7F] = 0x7E  # NaN codes -> +-448
    return c


def rand_scales(rng, shape):
    # log-uniform over ~20 binades so rounding lands everywhere
    return (2.0 ** rng.uniform(-12, 8, size=shape)).astype(np.float32)


# ---------------------------------------------------------------- decode ---

def test_decode_all_256_codes_match_torch():
    t = oracle.e4m3_table()
    ref = X.torch_decode(np.arange(256, dtype=np.uint8))
    nan_o, nan_r = np.isnan(t), np.isnan(ref)
    assert np.array_equal(nan_o, nan_r)
    assert np.flatnonzero(nan_o).tolist() == [0x7F, 0xFF]
    assert np.array_equal(t[~nan_o], ref[~nan_r])
    assert np.array_equal(np.signbit(t[~nan_o]), np.signbit(ref[~nan_r]))


def test_decode_special_values():
    t = oracle.e4m3_table()
    assert t[0x7E] == 448.0 and t[0xFE] == -448.0          # largest finite
    assert t[0x01] == 2.0 ** -9                            # smallest subnormal
    assert t[0x08] == 2.0 ** -6                            # smallest normal
    assert t[0x38] == 1.0
    assert t[0x80] == 0.0 and np.signbit(t[0x80])          # -0
    assert np.all(np.isfinite(np.delete(t, [0x7F, 0xFF])))  # no infinities
    # every finite value is a multiple of 2^-9 (basis of the exact block sums)
    f = t[np.isfinite(t)] * 512.0
    assert np.array_equal(f, np.round(f))


# -------------------------------------------------------------- rounding ---

def test_round_bf16_matches_torch_on_fp32_values():
    rng = np.random.default_rng(1)
    with np.errstate(over="ignore"):
        x = (rng.standard_normal(200000) * 2.0 ** rng.integers(-140, 128, 200000)).astype(np.float32)
    # exact ties: a bf16 value plus half its ulp (representable in fp32)
    base = rng.integers(0x0080, 0x7F00, 5000).astype(np.uint32) << 16
    ties = (base | 0x8000).view(np.float32)
    x = np.concatenate([x, ties, -ties, np.float32([0.0, -0.0, 1e-45, 3.3e38, -3.4e38])])
    x = x[np.isfinite(x)]
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.uint16).numpy()
    got = oracle.round_bf16(x.astype(np.float64))
    assert np.array_equal(got, ref)


def test_round_bf16_fp64_brute_force():
    """Values with more bits than fp32 holds, near ties, subnormals, overflow."""
    rng = np.random.default_rng(2)
    vals = list(rng.standard_normal(400) * 2.0 ** rng.integers(-135, 127, 400))
    bits, tbl = X._bf16_positive_table()
    for idx in rng.integers(1, len(tbl) - 2, 200):
        mid = (tbl[idx] + tbl[idx + 1]) / 2.0  # exact in fp64
        vals += [mid, np.nextafter(mid, np.inf), np.nextafter(mid, -np.inf)]
    big = float(tbl[-1])
    over_mid = big + (2.0 ** 128 - big) / 2
    vals += [big, over_mid, np.nextafter(over_mid, 0.0), 2.0 ** -134, 2.0 ** -133 * 1.5,
             3 * 2.0 ** -134]
    vals = np.array(vals + [-v for v in vals], dtype=np.float64)
    got = oracle.round_bf16(vals)
    for v, g in zip(vals, got):
        assert int(g) == X.round_bf16_exact(Fraction(float(v))), v


def test_round_f32_matches_numpy():
    rng = np.random.default_rng(3)
    x = rng.standard_normal(100000) * 2.0 ** rng.integers(-160, 128, 100000)
    with np.errstate(over="ignore"):
        ref = x.astype(np.float32)
    assert np.array_equal(oracle.round_f32(x), ref)


# ------------------------------------------------------------ block sums ---

def test_block_sums_fp64_equal_int64_route():
    rng = np.random.default_rng(4)
    a = rand_codes(rng, (9, 384))
    b = rand_codes(rng, (13, 384))
    a[0] = 0x7E  # +448 everywhere: largest block sum 128*448^2
    b[0] = 0x7E
    f = oracle.block_sums_f64(a, b)
    i, nan_seen = oracle.block_sums_i64(a, b)
    assert not nan_seen
    assert np.array_equal(f, i.astype(np.float64) * 2.0 ** -18)
    assert f[0, 0, 0] == 128 * 448.0 ** 2


def test_block_sums_int64_route_flags_nan():
    a = np.full((1, 128), 0x38, np.uint8)
    b = a.copy()
    b[0, 5] = 0xFF
    assert oracle.block_sums_i64(a, b)[1]


def test_block_sums_match_independent_integer_sums():
    rng = np.random.default_rng(5)
    a, b = rand_codes(rng, (4, 256)), rand_codes(rng, (6, 256))
    P = X.block_sums_int(a, b).astype(np.int64)
    i, _ = oracle.block_sums_i64(a, b)
    assert np.array_equal(P, i)


# ------------------------------------------------- dense vs exact values ---

@pytest.mark.parametrize("m,n,k", [(1, 1, 128), (3, 5, 256), (8, 17, 384), (17, 130, 256)])
def test_dense_matches_exact_rational(m, n, k):
    rng = np.random.default_rng(100 + m * n)
    a, b = rand_codes(rng, (m, k)), rand_codes(rng, (n, k))
    sa = rand_scales(rng, (m, k // 128))
    sb = rand_scales(rng, ((n + 127) // 128, k // 128))
    c, x = oracle.gemm_fp8_nt(a, sa, b, sb)
    sb_rows = [j // 128 for j in range(n)]
    ex = X.exact_elements(a, sa, b, sb, sb_rows)
    terms = X.abs_terms(a, sa, b, sb, sb_rows)
    for i in range(m):
        for j in range(n):
            e = ex[i][j]
            assert abs(Fraction(float(x[i, j])) - e) <= Fraction(2.0 ** -50) * Fraction(float(terms[i, j]))
            if not X.near_tie_bf16(e):
                assert int(c[i, j]) == X.round_bf16_exact(e), (i, j)


def test_dense_matches_numpy_fp64_matmul():
    rng = np.random.default_rng(6)
    m, n, k = 40, 300, 640
    a, b = rand_codes(rng, (m, k)), rand_codes(rng, (n, k))
    sa = rand_scales(rng, (m, k // 128))
    sb = rand_scales(rng, ((n + 127) // 128, k // 128))
    _, x = oracle.gemm_fp8_nt(a, sa, b, sb)
    A = X.torch_decode(a) * np.repeat(sa.astype(np.float64), 128, axis=1)      # exact
    Bs = np.repeat(np.repeat(sb.astype(np.float64), 128, axis=0)[:n], 128, axis=1)
    B = X.torch_decode(b) * Bs                                               # exact
    ref = A @ B.T
    bound = 1e-12 * (np.abs(A) @ np.abs(B).T)
    assert np.all(np.abs(x - ref) <= bound)


def test_dense_closed_form_all_ones():
    for k in (128, 7168):
        a = np.full((3, k), 0x38, np.uint8)
        b = np.full((5, k), 0x38, np.uint8)
        c, x = oracle.gemm_fp8_nt(a, np.ones((3, k // 128), np.float32), b,
                                  np.ones((1, k // 128), np.float32))
        assert np.all(x == k)
        assert np.all(oracle.bf16_to_f32(c) == k)  # k is exact in bf16


def test_dense_power_of_two_scale_and_negation_are_exact():
    rng = np.random.default_rng(7)
    m, n, k = 7, 150, 384
    a, b = rand_codes(rng, (m, k)), rand_codes(rng, (n, k))
    sa, sb = rand_scales(rng, (m, 3)), rand_scales(rng, (2, 3))
    c, x = oracle.gemm_fp8_nt(a, sa, b, sb)
    c2, x2 = oracle.gemm_fp8_nt(a, sa * np.float32(4.0), b, sb)
    assert np.array_equal(x2, 4.0 * x)
    assert np.array_equal(oracle.bf16_to_f32(c2), 4.0 * oracle.bf16_to_f32(c))
    cn, xn = oracle.gemm_fp8_nt(a ^ np.uint8(0x80), sa, b, sb)
    assert np.array_equal(xn, -x)
    assert np.array_equal(cn ^ np.uint16(0x8000), c)


def test_dense_k_block_permutation():
    rng = np.random.default_rng(8)
    m, n, k = 5, 20, 512
    a, b = rand_codes(rng, (m, k)), rand_codes(rng, (n, k))
    sa, sb = rand_scales(rng, (m, 4)), rand_scales(rng, (1, 4))
    _, x = oracle.gemm_fp8_nt(a, sa, b, sb)
    perm = np.array([2, 0, 3, 1])
    cols = np.concatenate([np.arange(p * 128, (p + 1) * 128) for p in perm])
    _, xp = oracle.gemm_fp8_nt(a[:, cols], sa[:, perm], b[:, cols], sb[:, perm])
    terms = X.abs_terms(a, sa, b, sb, [0] * n)
    assert np.all(np.abs(xp - x) <= 1e-14 * terms)


def test_dense_n_tail_uses_ceil_div_scale_rows():
    """N=130: columns 128,129 use sb row 1; changing sb row 1 moves only them."""
    rng = np.random.default_rng(9)
    a, b = rand_codes(rng, (4, 256)), rand_codes(rng, (130, 256))
    sa, sb = rand_scales(rng, (4, 2)), rand_scales(rng, (2, 2))
    _, x = oracle.gemm_fp8_nt(a, sa, b, sb)
    sb2 = sb.copy()
    sb2[1] *= 2
    _, x2 = oracle.gemm_fp8_nt(a, sa, b, sb2)
    assert np.array_equal(x2[:, :128], x[:, :128])
    assert np.array_equal(x2[:, 128:], 2 * x[:, 128:])


def test_sampled_dense_equals_full():
    rng = np.random.default_rng(10)
    m, n, k = 33, 260, 256
    a, b = rand_codes(rng, (m, k)), rand_codes(rng, (n, k))
    sa, sb = rand_scales(rng, (m, 2)), rand_scales(rng, (3, 2))
    _, x = oracle.gemm_fp8_nt(a, sa, b, sb)
    rows, cols = rng.integers(0, m, 500), rng.integers(0, n, 500)
    assert np.array_equal(oracle.gemm_fp8_nt_at(a, sa, b, sb, rows, cols), x[rows, cols])


# ------------------------------------------------------------- contiguous ---

def _contig_case(rng, g=3, seg=128, n=70, k=256, ids=None):
    m_total = g * seg
    a = rand_codes(rng, (m_total, k))
    sa = rand_scales(rng, (m_total, k // 128))
    b = rand_codes(rng, (g, n, k))
    sb = rand_scales(rng, (g, (n + 127) // 128, k // 128))
    if ids is None:
        ids = np.full(m_total, -1, np.int32)
        for e in range(g):
            v = seg - int(rng.integers(0, seg // 2))
            ids[e * seg:e * seg + v] = e
    return a, sa, b, sb, ids


def test_contiguous_matches_exact_rational():
    rng = np.random.default_rng(11)
    g, n, k = 3, 9, 256
    ids = np.array([0, 2, -1, 1, 1, 0, 3, -1, 2], np.int32)  # unsorted, -1 and an id >= g
    m = ids.size
    a, b = rand_codes(rng, (m, k)), rand_codes(rng, (g, n, k))
    sa, sb = rand_scales(rng, (m, 2)), rand_scales(rng, (g, 1, 2))
    sentinel = np.full((m, n), 0xFFFF, np.uint16)
    c, _ = oracle.grouped_contiguous(a, sa, b, sb, ids, sentinel)
    for r in range(m):
        e = ids[r]
        if e < 0 or e >= g:
            assert np.all(c[r] == 0xFFFF)
            continue
        ex = X.exact_elements(a[r:r + 1], sa[r:r + 1], b[e], sb[e], [0] * n)
        for j in range(n):
            if not X.near_tie_bf16(ex[0][j]):
                assert int(c[r, j]) == X.round_bf16_exact(ex[0][j])


def test_contiguous_equals_dense_per_segment_and_padding_untouched():
    rng = np.random.default_rng(12)
    a, sa, b, sb, ids = _contig_case(rng)
    m_total, n = ids.size, b.shape[1]
    sentinel = np.full((m_total, n), 0xFFFF, np.uint16)
    c, x = oracle.grouped_contiguous(a, sa, b, sb, ids, sentinel)
    for e in range(b.shape[0]):
        rows = np.flatnonzero(ids == e)
        cd, xd = oracle.gemm_fp8_nt(a[rows], sa[rows], b[e], sb[e])
        assert np.array_equal(c[rows], cd) and np.array_equal(x[rows], xd)
    pad = ids < 0
    assert pad.any() and np.all(c[pad] == 0xFFFF)


def test_contiguous_group_independence():
    rng = np.random.default_rng(13)
    a, sa, b, sb, ids = _contig_case(rng)
    init = np.zeros((ids.size, b.shape[1]), np.uint16)
    c, _ = oracle.grouped_contiguous(a, sa, b, sb, ids, init)
    b2 = b.copy()
    b2[1] = rand_codes(rng, b[1].shape)
    c2, _ = oracle.grouped_contiguous(a, sa, b2, sb, ids, init)
    changed = np.any(c2 != c, axis=1)
    assert np.all(ids[changed] == 1) and changed[ids == 1].any()


def test_contiguous_sampled_equals_full():
    rng = np.random.default_rng(14)
    a, sa, b, sb, ids = _contig_case(rng)
    _, x = oracle.grouped_contiguous(a, sa, b, sb, ids, np.zeros((ids.size, b.shape[1]), np.uint16))
    rows, cols = rng.integers(0, ids.size, 400), rng.integers(0, b.shape[1], 400)
    v, w = oracle.grouped_contiguous_at(a, sa, b, sb, ids, rows, cols)
    assert np.array_equal(w, ids[rows] >= 0)
    assert np.array_equal(v[w], x[rows, cols][w])


# ----------------------------------------------------------------- masked ---

def test_masked_matches_exact_and_clamps():
    rng = np.random.default_rng(15)
    g, m_max, n, k = 5, 6, 10, 256
    masked_m = np.array([0, 1, 6, 9, -3], np.int32)  # empty, one, full, > m_max, negative
    a = rand_codes(rng, (g, m_max, k))
    sa = rand_scales(rng, (g, m_max, 2))
    b = rand_codes(rng, (g, n, k))
    sb = rand_scales(rng, (g, 1, 2))
    sentinel = np.full((g, m_max, n), 0xFFFF, np.uint16)
    c, _ = oracle.grouped_masked(a, sa, b, sb, masked_m, sentinel)
    for gi in range(g):
        v = min(max(int(masked_m[gi]), 0), m_max)
        assert np.all(c[gi, v:] == 0xFFFF)
        if v:
            ex = X.exact_elements(a[gi, :v], sa[gi, :v], b[gi], sb[gi], [0] * n)
            for r in range(v):
                for j in range(n):
                    if not X.near_tie_bf16(ex[r][j]):
                        assert int(c[gi, r, j]) == X.round_bf16_exact(ex[r][j])


def test_masked_equals_dense_on_prefix_and_group_independence():
    rng = np.random.default_rng(16)
    g, m_max, n, k = 3, 40, 140, 384
    masked_m = np.array([17, 40, 3], np.int32)
    a = rand_codes(rng, (g, m_max, k))
    sa = rand_scales(rng, (g, m_max, 3))
    b = rand_codes(rng, (g, n, k))
    sb = rand_scales(rng, (g, 2, 3))
    init = np.zeros((g, m_max, n), np.uint16)
    c, x = oracle.grouped_masked(a, sa, b, sb, masked_m, init)
    for gi in range(g):
        v = masked_m[gi]
        cd, xd = oracle.gemm_fp8_nt(a[gi, :v], sa[gi, :v], b[gi], sb[gi])
        assert np.array_equal(c[gi, :v], cd) and np.array_equal(x[gi, :v], xd)
    b2 = b.copy()
    b2[2] ^= np.uint8(0x80)
    c2, _ = oracle.grouped_masked(a, sa, b2, sb, masked_m, init)
    assert np.array_equal(c2[:2], c[:2]) and not np.array_equal(c2[2], c[2])
    groups = rng.integers(0, g, 300)
    rows, cols = rng.integers(0, m_max, 300), rng.integers(0, n, 300)
    vals, wr = oracle.grouped_masked_at(a, sa, b, sb, masked_m, groups, rows, cols)
    assert np.array_equal(wr, rows < masked_m[groups])
    assert np.array_equal(vals[wr], x[groups, rows, cols][wr])


# ------------------------------------------------------------------ wgrad ---

def test_wgrad_matches_exact_rational_fp32():
    rng = np.random.default_rng(17)
    m, n, k = 4, 6, 384
    a, b = rand_codes(rng, (m, k)), rand_codes(rng, (n, k))
    sa, sb = rand_scales(rng, (m, 3)), rand_scales(rng, (n, 3))  # per-row scales on both
    d0 = rng.standard_normal((m, n)).astype(np.float32)
    d, _ = oracle.wgrad(a, sa, b, sb, d0)
    ex = X.exact_elements(a, sa, b, sb, list(range(n)))
    for i in range(m):
        for j in range(n):
            assert d[i, j] == X.round_f32_exact(Fraction(float(d0[i, j])) + ex[i][j])


def test_wgrad_accumulates_and_differs_from_block_scaled_dense():
    rng = np.random.default_rng(18)
    m, n, k = 12, 140, 256
    a, b = rand_codes(rng, (m, k)), rand_codes(rng, (n, k))
    sa, sb = rand_scales(rng, (m, 2)), rand_scales(rng, (n, 2))
    d_zero, x_zero = oracle.wgrad(a, sa, b, sb, np.zeros((m, n), np.float32))
    d0 = rng.standard_normal((m, n)).astype(np.float32)
    _, x = oracle.wgrad(a, sa, b, sb, d0)
    assert np.allclose(x - d0, x_zero, rtol=0, atol=1e-9 * (np.abs(x_zero).max() + 1))
    assert np.array_equal(d_zero, x_zero.astype(np.float32))
    # per-row sb that is constant within each 128-row block == dense block scaling
    sbb = rand_scales(rng, (2, 2))
    _, xd = oracle.gemm_fp8_nt(a, sa, b, sbb)
    _, xw = oracle.wgrad(a, sa, b, np.repeat(sbb, 128, axis=0)[:n], np.zeros((m, n), np.float32))
    assert np.array_equal(xd, xw)


def test_k_grouped_wgrad_equals_wgrad_per_slice():
    rng = np.random.default_rng(19)
    m, n = 9, 33
    ks = [128, 0, 384, 256]
    t = sum(ks)
    a, b = rand_codes(rng, (m, t)), rand_codes(rng, (n, t))
    sa, sb = rand_scales(rng, (m, t // 128)), rand_scales(rng, (n, t // 128))
    d0 = rng.standard_normal((len(ks), m, n)).astype(np.float32)
    d, x = oracle.k_grouped_wgrad(a, sa, b, sb, ks, d0)
    o = 0
    for gi, kk in enumerate(ks):
        if kk == 0:
            assert np.array_equal(d[gi], d0[gi])
        else:
            sl = slice(o, o + kk)
            bl = slice(o // 128, (o + kk) // 128)
            dg, xg = oracle.wgrad(a[:, sl], sa[:, bl], b[:, sl], sb[:, bl], d0[gi])
            assert np.array_equal(d[gi], dg) and np.array_equal(x[gi], xg)
        o += kk
    groups, rows, cols = rng.integers(0, 4, 200), rng.integers(0, m, 200), rng.integers(0, n, 200)
    v = oracle.k_grouped_wgrad_at(a, sa, b, sb, ks, d0, groups, rows, cols)
    assert np.array_equal(v, x[groups, rows, cols])
    v1 = oracle.wgrad_at(a, sa, b, sb, d0[0], rows, cols)
    _, x1 = oracle.wgrad(a, sa, b, sb, d0[0])
    assert np.array_equal(v1, x1[rows, cols])


def test_k_grouped_wgrad_matches_exact_rational():
    rng = np.random.default_rng(20)
    m, n = 3, 4
    ks = [256, 128]
    t = sum(ks)
    a, b = rand_codes(rng, (m, t)), rand_codes(rng, (n, t))
    sa, sb = rand_scales(rng, (m, 3)), rand_scales(rng, (n, 3))
    d0 = rng.standard_normal((2, m, n)).astype(np.float32)
    d, _ = oracle.k_grouped_wgrad(a, sa, b, sb, ks, d0)
    for gi, (lo, hi) in enumerate([(0, 2), (2, 3)]):
        ex = X.exact_elements(a, sa, b, sb, list(range(n)), lo, hi)
        for i in range(m):
            for j in range(n):
                assert d[gi, i, j] == X.round_f32_exact(Fraction(float(d0[gi, i, j])) + ex[i][j])


def test_invalid_arguments_rejected():
    a = np.zeros((2, 100), np.uint8)
    with pytest.raises(ValueError):
        oracle.gemm_fp8_nt(a, np.ones((2, 1), np.float32), a, np.ones((1, 1), np.float32))
    with pytest.raises(ValueError):
        oracle.k_grouped_wgrad(np.zeros((2, 256), np.uint8), np.ones((2, 2), np.float32),
                               np.zeros((2, 256), np.uint8), np.ones((2, 2), np.float32),
                               [100, 156], np.zeros((2, 2, 2), np.float32))


# ------------------------------------------------- page-printed shapes pin ---

def test_usage_example_shapes_golden():
    """The pages' usage example pairs M=4096,N=2112,K=7168 with scale tensors
    [4096,56] and [17,56]: K/128 blocks and ceil(N/128) weight row blocks."""
    with open(os.path.join(GOLDEN, "usage_example_shapes.json")) as f:
        gold = json.load(f)
    m, n, k = gold["m"], gold["n"], gold["k"]
    rng = np.random.default_rng(21)
    a, sa = inputs.quantize_1x128(rng.standard_normal((m, 256)).astype(np.float32))
    assert sa.shape == (m, 2)
    x = np.zeros((n, k), np.float32)
    x[::97, ::131] = 1.0
    b, sb = inputs.quantize_128x128(x)
    assert list(sb.shape) == gold["rhs_scale_shape"]
    assert list(b.shape) == gold["rhs_shape"]
    assert k // 128 == gold["lhs_scale_shape"][1]
    # the oracle reads sb row 16 for columns 2048..2111
    a1 = np.full((1, k), 0x38, np.uint8)
    sa1 = np.ones((1, k // 128), np.float32)
    b1 = np.full((n, k), 0x38, np.uint8)
    sb1 = np.ones((17, k // 128), np.float32)
    sb1[16] = 2.0
    cols = np.array([0, 2047, 2048, 2111])
    v = oracle.gemm_fp8_nt_at(a1, sa1, b1, sb1, np.zeros(4, np.int64), cols)
    assert v.tolist() == [k, k, 2 * k, 2 * k]


# --------------------------------------------------------- harness pins ---

def test_harness_is_deterministic_and_quantiser_bounds():
    d1 = inputs.make_dense(64, 130, 256, seed=inputs.SEED_BASE)
    d2 = inputs.make_dense(64, 130, 256, seed=inputs.SEED_BASE)
    for f in ("a", "sa", "b", "sb"):
        assert np.array_equal(getattr(d1, f), getattr(d2, f))
    h = hashlib.sha256(d1.a.tobytes() + d1.b.tobytes() + d1.sa.tobytes() + d1.sb.tobytes()).hexdigest()
    assert h == HARNESS_HASH, h
    vals = X.torch_decode(d1.a)
    assert np.all(np.isfinite(vals)) and np.abs(vals).max() == 448.0
    # each 1x128 group reaches 448 in magnitude exactly once scaled by absmax/448
    g = np.abs(vals).reshape(64, 2, 128).max(axis=2)
    assert np.all(g == 448.0)


HARNESS_HASH = "b8f626aff7f5e00b6a9b799e66ff1af040b22a61646662bdb07e77afbfdc5cdc"
