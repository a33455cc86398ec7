"""The allocation-free masked entry point (dg_grouped_fp8_masked_noalloc)
against the default one (dg_grouped_fp8_masked) through the C ABI: two calls
in a row, the second on a smaller problem, must give the same bits as the
default entry point and match the oracle; the call keeps its K split under
HIP graph capture (the default one drops it there) and every replay with new
masked_m matches the eager default result; a call whose split-K partials
exceed the scratch is rejected before anything is enqueued."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from harness import inputs
from tests.parity import SENTINEL_BF16, bf16_bits, bits_to_f64, check_close, dev, say, sentinel_bf16

pytestmark = pytest.mark.gpu

WORKSPACE = 4  # DG_ERROR_WORKSPACE


@pytest.fixture(scope="module")
def dg():
    import moe_grouped_gemm_x128_amd as m
    return m


def _operands(x):
    return (dev(x.a).view(torch.float8_e4m3fn), dev(x.sa), dev(x.b).view(torch.float8_e4m3fn), dev(x.sb),
            dev(x.masked_m))


def _sampled_check(x, bits, what, count=1024):
    """Sampled outputs of the valid rows against the oracle, and the sentinel
    bits of every row past masked_m."""
    rng = np.random.default_rng(5)
    valid = np.clip(x.masked_m, 0, x.m_max)
    groups = [g for g in range(x.g) if valid[g] > 0]
    if groups:
        gs = rng.choice(groups, count)
        rows = np.array([rng.integers(0, valid[g]) for g in gs], np.int64)
        cols = rng.integers(0, x.n, count)
        vals, wr = oracle.grouped_masked_at(x.a, x.sa, x.b, x.sb, x.masked_m, gs, rows, cols)
        assert wr.all()
        ref = oracle.round_bf16(vals)
        check_close(bits_to_f64(bits[gs, rows, cols]), bits_to_f64(ref), what)
    for g in range(x.g):
        assert np.all(bits[g, valid[g]:] == SENTINEL_BF16), f"{what}: group {g} rows past masked_m written"
        assert not np.any(bits[g, :valid[g]] == SENTINEL_BF16), f"{what}: group {g} valid rows not written"


def test_noalloc_matches_default_two_calls(dg):
    """Two calls in a row (the second smaller), each against the default entry
    point's bits and the oracle."""
    for i, (g, n, k) in enumerate([(2, 4096, 7168), (1, 1024, 4608)]):
        x = inputs.make_masked(g, 256, n, k, seed=inputs.SEED_BASE + 90 + i)
        cfg = dg.select_config(dg.KIND_MASKED, 256, n, k, g)
        say(f"noalloc call {i}: G={g} N={n} K={k} plan {cfg}")
        assert cfg["k_splits"] > 1, "the case must use the scratch"
        a, sa, b, sb, mm = _operands(x)
        c_ref, c_new = sentinel_bf16((g, 256, n)), sentinel_bf16((g, 256, n))
        dg.dg_grouped_fp8_masked(a, sa, b, sb, c_ref, mm)
        dg.dg_grouped_fp8_masked_noalloc(a, sa, b, sb, c_new, mm)
        torch.cuda.synchronize()
        ref_bits, new_bits = bf16_bits(c_ref), bf16_bits(c_new)
        assert np.array_equal(ref_bits, new_bits), f"call {i}: allocation-free result differs from the default"
        _sampled_check(x, new_bits, f"noalloc call {i}")


def test_noalloc_under_graph_capture(dg):
    """Captured with its K split; every replay with new masked_m and A equals
    the eager default call on the same inputs."""
    g, n, k = 1, 4096, 7168
    x = inputs.make_masked(g, 256, n, k, seed=inputs.SEED_BASE + 93)
    say("noalloc under graph capture G=1 N=4096 K=7168")
    a, sa, b, sb, mm = _operands(x)
    out = sentinel_bf16((g, 256, n))
    s = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        dg.dg_grouped_fp8_masked_noalloc(a, sa, b, sb, out, mm)
        torch.cuda.synchronize()
        with torch.cuda.graph(graph, stream=s):
            dg.dg_grouped_fp8_masked_noalloc(a, sa, b, sb, out, mm)
    torch.cuda.synchronize()
    for rep, m in enumerate([192, 1, 256, 300, 0, 97]):
        y = inputs.make_masked(g, 256, n, k, seed=inputs.SEED_BASE + 94 + rep, masked_m=[m])
        a.copy_(dev(y.a).view(torch.float8_e4m3fn))
        sa.copy_(dev(y.sa))
        mm.copy_(dev(y.masked_m))
        out.view(torch.int16).fill_(-1)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        ref = sentinel_bf16((g, 256, n))
        dg.dg_grouped_fp8_masked(a, sa, b, sb, ref, mm)
        torch.cuda.synchronize()
        assert np.array_equal(bf16_bits(out), bf16_bits(ref)), f"replay {rep} (masked_m={m}) differs from eager"
        if rep < 2:
            y.b, y.sb = x.b, x.sb
            _sampled_check(y, bf16_bits(out), f"noalloc replay {rep}")


def test_noalloc_rejects_oversized_partials(dg, monkeypatch):
    """K split 14 ways (16 asked, 4-block chunks of 56) for G=2 x 256 rows x
    N=4096 needs 14 x 8 MB of partials, more than the 64 MB scratch:
    rejected, nothing written."""
    monkeypatch.setenv("DG_FORCE_SPLITS", "16")
    x = inputs.make_masked(2, 256, 4096, 7168, seed=inputs.SEED_BASE + 99)
    a, sa, b, sb, mm = _operands(x)
    out = sentinel_bf16((2, 256, 4096))
    say("noalloc oversized partials")
    st = dg._lib.dg_grouped_fp8_masked_noalloc(a.data_ptr(), sa.data_ptr(), b.data_ptr(), sb.data_ptr(),
                                               out.data_ptr(), mm.data_ptr(), 2, 256, 4096, 7168,
                                               torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert st == WORKSPACE
    assert np.all(bf16_bits(out) == SENTINEL_BF16)
