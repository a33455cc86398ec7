"""GPU parity of the dense BF16 NT GEMM against the CPU oracle
(dgo_gemm_bf16_nt): every output at small sizes over every tile instance,
ragged tails, N not a multiple of 4 and forced K splits; sampled outputs at a
full workload size in the benchmark's launch configuration.  The bar is the
library's: |gpu - ref| <= 2^-7 |ref| + 1e-3 max|ref| per element and a
relative Frobenius error <= 2e-3."""
from __future__ import annotations

import os

import numpy as np
import pytest
import torch

import oracle
from harness import inputs
from tests.parity import bf16_bits, bits_to_f64, check_close, say, sentinel_bf16

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


def bf16_dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def run(dg, d):
    c = sentinel_bf16((d.m, d.n))
    dg.dg_gemm_bf16_nt(bf16_dev(d.a), bf16_dev(d.b), c)
    torch.cuda.synchronize()
    return bf16_bits(c)


@pytest.mark.parametrize("tile", TILES)
@pytest.mark.parametrize("m,n,k", [(1, 1, 64), (17, 130, 128), (257, 390, 448), (64, 2112, 1024),
                                   (300, 1000, 192), (129, 18, 640)])
def test_bf16_ragged(dg, force, m, n, k, tile):
    d = inputs.make_dense_bf16(m, n, k, seed=inputs.SEED_BASE + 61 + m + n)
    force(tile)
    say(f"bf16 {m}x{n}x{k} tile={tile}")
    got = run(dg, d)
    ref, _ = oracle.gemm_bf16_nt(d.a, d.b)
    check_close(bits_to_f64(got), bits_to_f64(ref), f"bf16 {m}x{n}x{k} {tile}")
    assert np.array_equal(got, run(dg, d)), "not deterministic"


@pytest.mark.parametrize("splits", [2, 5])
def test_bf16_split_k(dg, force, splits):
    d = inputs.make_dense_bf16(64, 500, 2048, seed=inputs.SEED_BASE + 62)
    force("64x64x1x4", splits)
    say(f"bf16 64x500x2048 splits={splits}")
    got = run(dg, d)
    ref, _ = oracle.gemm_bf16_nt(d.a, d.b)
    check_close(bits_to_f64(got), bits_to_f64(ref), f"bf16 split {splits}")


def test_bf16_exact_integers(dg):
    """Small-integer operands: every partial sum is exact in fp32, so the GPU
    result equals the oracle's bit for bit."""
    rng = np.random.default_rng(63)
    m, n, k = 130, 200, 512
    to = lambda x: torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    d = inputs.DenseBf16(m, n, k, to(rng.integers(-8, 9, (m, k))), to(rng.integers(-8, 9, (n, k))))
    say("bf16 exact integers")
    got = run(dg, d)
    ref, _ = oracle.gemm_bf16_nt(d.a, d.b)
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("m,n,k", [(4096, 7168, 16384), (64, 7168, 16384), (4096, 2112, 7168)])
def test_bf16_full_size_sampled(dg, m, n, k):
    d = inputs.make_dense_bf16(m, n, k, seed=inputs.SEED_BASE + 1)
    say(f"bf16 full {m}x{n}x{k}")
    got = run(dg, d)
    rng = np.random.default_rng(m + n + k + 1)
    rows = list(rng.integers(0, m, 1536)) + [0, m - 1, 0, m - 1]
    cols = list(rng.integers(0, n, 1536)) + [0, n - 1, n - 1, 0]
    rows, cols = np.array(rows, np.int64), np.array(cols, np.int64)
    ref = oracle.round_bf16(oracle.gemm_bf16_nt_at(d.a, d.b, rows, cols))
    check_close(bits_to_f64(got[rows, cols]), bits_to_f64(ref), f"bf16 full {m}x{n}x{k}")
    assert not np.any(got == 0xFFFF), "outputs left unwritten"
