"""GPU parity of the dense GEMM with power-of-two (UE8M0) scales, applied by
the block-scaled MFMA, against the CPU oracle.  A power-of-two scale is a
special case of the oracle's fp32 scales, so the oracle is the same function
and the bar is the same as for dg_gemm_fp8_nt: every output at small sizes
over every tile instance, ragged tails, N not a multiple of 4 and forced K
splits; sampled outputs at a full workload size in the benchmark's launch
configuration.  The packed format (int32 words of four exponent bytes) meets
the same bar against the oracle's unpack-then-GEMM, and is bit-identical to
the fp32-scale entry point on the same scales; the packer fills the bytes
past the last K block with the NaN code, so reading one would show."""
from __future__ import annotations

import os

import numpy as np
import pytest
import torch

import oracle
from harness import inputs
from tests.parity import bf16_bits, bits_to_f64, check_close, dev, say, sentinel_bf16

pytestmark = pytest.mark.gpu

TILES = [None, "256x256x2x4", "256x256x1x8", "256x224x4x2", "256x128x2x2", "128x128x2x2", "128x64x2x2",
         "64x128x1x4", "64x64x1x4", "64x32x2x2"]


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


def run(dg, d):
    c = sentinel_bf16((d.m, d.n))
    dg.dg_gemm_fp8_nt_ue8m0(dev(d.a), dev(d.sa), dev(d.b), dev(d.sb), c)
    torch.cuda.synchronize()
    return bf16_bits(c)


def test_harness_scales_are_powers_of_two():
    d = inputs.make_dense(70, 300, 384, seed=inputs.SEED_BASE + 50, pow2=True)
    for s in (d.sa, d.sb):
        m, _ = np.frexp(s)
        assert np.all(m == 0.5)


@pytest.mark.parametrize("tile", TILES)
@pytest.mark.parametrize("m,n,k", [(1, 1, 128), (17, 130, 128), (257, 390, 384), (64, 2112, 1024),
                                   (300, 1000, 256), (129, 18, 640)])
def test_ue8m0_ragged(dg, force, m, n, k, tile):
    d = inputs.make_dense(m, n, k, seed=inputs.SEED_BASE + 51 + m + n, pow2=True)
    force(tile)
    say(f"ue8m0 {m}x{n}x{k} tile={tile}")
    got = run(dg, d)
    ref, _ = oracle.gemm_fp8_nt(d.a, d.sa, d.b, d.sb)
    check_close(bits_to_f64(got), bits_to_f64(ref), f"ue8m0 {m}x{n}x{k} {tile}")
    assert np.array_equal(got, run(dg, d)), "not deterministic"


@pytest.mark.parametrize("splits", [2, 3, 7])
def test_ue8m0_split_k(dg, force, splits):
    d = inputs.make_dense(64, 500, 1792, seed=inputs.SEED_BASE + 52, pow2=True)
    force("64x64x1x4", splits)
    say(f"ue8m0 64x500x1792 splits={splits}")
    got = run(dg, d)
    ref, _ = oracle.gemm_fp8_nt(d.a, d.sa, d.b, d.sb)
    check_close(bits_to_f64(got), bits_to_f64(ref), f"ue8m0 split {splits}")


def test_ue8m0_scale_range(dg):
    """Random codes with scales 2^e over e in [-60, 40] (the scale byte E runs
    over most of its range; products stay within fp32)."""
    rng = np.random.default_rng(53)
    m, n, k = 200, 260, 512
    a = rng.integers(0, 256, (m, k), dtype=np.uint8)
    b = rng.integers(0, 256, (n, k), dtype=np.uint8)
    a[(a & 0x7F) == 0x7F] = 0x7E
    b[(b & 0x7F) == 0x7F] = 0x7E
    sa = np.ldexp(1.0, rng.integers(-60, 40, (m, k // 128))).astype(np.float32)
    sb = np.ldexp(1.0, rng.integers(-60, 40, ((n + 127) // 128, k // 128))).astype(np.float32)
    d = inputs.Dense(m, n, k, a, sa, b, sb)
    say("ue8m0 scale range")
    got = run(dg, d)
    ref, _ = oracle.gemm_fp8_nt(a, sa, b, sb)
    check_close(bits_to_f64(got), bits_to_f64(ref), "ue8m0 scale range")


def test_ue8m0_agrees_with_fp32_scale_path(dg):
    """On power-of-two scales both dense entry points meet the oracle's bar."""
    d = inputs.make_dense(512, 768, 2048, seed=inputs.SEED_BASE + 54, pow2=True)
    say("ue8m0 vs fp32-scale path")
    got = run(dg, d)
    c = sentinel_bf16((d.m, d.n))
    dg.dg_gemm_fp8_nt(dev(d.a), dev(d.sa), dev(d.b), dev(d.sb), c)
    torch.cuda.synchronize()
    ref, _ = oracle.gemm_fp8_nt(d.a, d.sa, d.b, d.sb)
    check_close(bits_to_f64(got), bits_to_f64(ref), "ue8m0")
    check_close(bits_to_f64(bf16_bits(c)), bits_to_f64(ref), "fp32-scale path")


@pytest.mark.parametrize("m,n,k", [(4096, 7168, 16384), (64, 7168, 16384), (4096, 2112, 7168)])
def test_ue8m0_full_size_sampled(dg, m, n, k):
    """Full workload sizes in the library's own launch configuration; the
    oracle computes sampled outputs (corners, tails, scale-block edges)."""
    d = inputs.make_dense(m, n, k, seed=inputs.SEED_BASE + 1, pow2=True)
    say(f"ue8m0 full {m}x{n}x{k}")
    got = run(dg, d)
    rng = np.random.default_rng(m + n + k)
    rows = list(rng.integers(0, m, 1536)) + [0, m - 1, 0, m - 1]
    cols = list(rng.integers(0, n, 1536)) + [0, n - 1, n - 1, 0]
    for c0 in (127, 128, n - 64, n - 1):
        rows.append(int(rng.integers(0, m)))
        cols.append(c0)
    rows, cols = np.array(rows, np.int64), np.array(cols, np.int64)
    ref_bits = oracle.round_bf16(oracle.gemm_fp8_nt_at(d.a, d.sa, d.b, d.sb, rows, cols))
    check_close(bits_to_f64(got[rows, cols]), bits_to_f64(ref_bits), f"ue8m0 full {m}x{n}x{k}")
    assert not np.any(got == 0xFFFF), "outputs left unwritten"


def run_packed(dg, d, sa_w=None, sb_w=None):
    sa_w = inputs.pack_ue8m0(d.sa) if sa_w is None else sa_w
    sb_w = inputs.pack_ue8m0(d.sb) if sb_w is None else sb_w
    c = sentinel_bf16((d.m, d.n))
    dg.dg_gemm_fp8_nt_ue8m0_packed(dev(d.a), dev(sa_w), dev(d.b), dev(sb_w), c)
    torch.cuda.synchronize()
    return bf16_bits(c)


@pytest.mark.parametrize("tile", [None, "256x256x2x4", "256x256x1x8", "128x128x2x2", "64x64x1x4", "64x32x2x2"])
@pytest.mark.parametrize("m,n,k", [(1, 1, 128), (17, 130, 384), (257, 390, 640), (129, 18, 1024),
                                   (300, 1000, 1152)])
def test_ue8m0_packed_ragged(dg, force, m, n, k, tile):
    """K blocks 1, 3, 5, 8, 9: whole and padded last words."""
    d = inputs.make_dense(m, n, k, seed=inputs.SEED_BASE + 61 + m + n, pow2=True)
    force(tile)
    say(f"ue8m0 packed {m}x{n}x{k} tile={tile}")
    got = run_packed(dg, d)
    bits, _ = oracle.gemm_fp8_nt_ue8m0_packed(d.a, inputs.pack_ue8m0(d.sa), d.b, inputs.pack_ue8m0(d.sb))
    check_close(bits_to_f64(got), bits_to_f64(bits), f"ue8m0 packed {m}x{n}x{k} {tile}")
    assert np.array_equal(got, run(dg, d)), "packed and fp32 power-of-two scales differ"


@pytest.mark.parametrize("splits", [2, 3, 7])
def test_ue8m0_packed_split_k(dg, force, splits):
    """Splits that start inside a scale word (14 K blocks over 3 or 7 splits)."""
    d = inputs.make_dense(64, 500, 1792, seed=inputs.SEED_BASE + 62, pow2=True)
    force("64x64x1x4", splits)
    say(f"ue8m0 packed 64x500x1792 splits={splits}")
    got = run_packed(dg, d)
    bits, _ = oracle.gemm_fp8_nt_ue8m0_packed(d.a, inputs.pack_ue8m0(d.sa), d.b, inputs.pack_ue8m0(d.sb))
    check_close(bits_to_f64(got), bits_to_f64(bits), f"ue8m0 packed split {splits}")
    assert np.array_equal(got, run(dg, d)), "packed and fp32 power-of-two scales differ"


def test_ue8m0_packed_scale_range(dg):
    """Exponent bytes over 67..167 (scales 2^-60 .. 2^40) in every byte lane."""
    rng = np.random.default_rng(63)
    m, n, k = 200, 260, 896
    a = rng.integers(0, 256, (m, k), dtype=np.uint8)
    b = rng.integers(0, 256, (n, k), dtype=np.uint8)
    a[(a & 0x7F) == 0x7F] = 0x7E
    b[(b & 0x7F) == 0x7F] = 0x7E
    sa = np.ldexp(1.0, rng.integers(-60, 40, (m, k // 128))).astype(np.float32)
    sb = np.ldexp(1.0, rng.integers(-60, 40, ((n + 127) // 128, k // 128))).astype(np.float32)
    d = inputs.Dense(m, n, k, a, sa, b, sb)
    say("ue8m0 packed scale range")
    got = run_packed(dg, d)
    bits, _ = oracle.gemm_fp8_nt_ue8m0_packed(a, inputs.pack_ue8m0(sa), b, inputs.pack_ue8m0(sb))
    check_close(bits_to_f64(got), bits_to_f64(bits), "ue8m0 packed scale range")


def test_ue8m0_packed_nan_code(dg):
    """The E8M0 NaN code (255) in one row's K block makes that row NaN and
    leaves every other row as the oracle gives it."""
    d = inputs.make_dense(70, 200, 512, seed=inputs.SEED_BASE + 64, pow2=True)
    sa_w = inputs.pack_ue8m0(d.sa)
    raw = sa_w.view(np.uint8).reshape(70, -1).copy()
    raw[5, 2] = 255                                   # row 5, K block 2
    sa_w = raw.view(np.int32).reshape(sa_w.shape)
    say("ue8m0 packed NaN code")
    got = run_packed(dg, d, sa_w=sa_w)
    vals = bits_to_f64(got)
    assert np.all(np.isnan(vals[5])), "row with the NaN code"
    bits, _ = oracle.gemm_fp8_nt_ue8m0_packed(d.a, sa_w, d.b, inputs.pack_ue8m0(d.sb))
    keep = np.arange(70) != 5
    check_close(vals[keep], bits_to_f64(bits)[keep], "ue8m0 packed other rows")


def test_ue8m0_packed_full_size_sampled(dg):
    """4096x7168x16384 (128 K blocks, 32 words per row) in the library's own
    launch configuration: bit-identical to the fp32-scale entry point
    everywhere, sampled outputs against the oracle."""
    m, n, k = 4096, 7168, 16384
    d = inputs.make_dense(m, n, k, seed=inputs.SEED_BASE + 1, pow2=True)
    say(f"ue8m0 packed full {m}x{n}x{k}")
    got = run_packed(dg, d)
    assert np.array_equal(got, run(dg, d)), "packed and fp32 power-of-two scales differ"
    rng = np.random.default_rng(65)
    rows = np.concatenate([rng.integers(0, m, 1024), [0, m - 1, 0, m - 1]]).astype(np.int64)
    cols = np.concatenate([rng.integers(0, n, 1024), [0, n - 1, n - 1, 0]]).astype(np.int64)
    ref_bits = oracle.round_bf16(oracle.gemm_fp8_nt_at(d.a, oracle.unpack_ue8m0(inputs.pack_ue8m0(d.sa), k // 128),
                                                      d.b, oracle.unpack_ue8m0(inputs.pack_ue8m0(d.sb), k // 128),
                                                      rows, cols))
    check_close(bits_to_f64(got[rows, cols]), bits_to_f64(ref_bits), "ue8m0 packed full")
