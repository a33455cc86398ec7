"""Entry points under HIP graph capture: the quantiser, the power-of-two-scale
GEMM and the BF16 GEMM, alone and as one captured quantise -> GEMM pipeline;
the masked and contiguous grouped GEMMs with their device-side control data
(masked_m, m_indices) rewritten between replays; and the contiguous GEMM with
the fused SwiGLU + re-quantise epilogue.  Each graph is replayed several times
with new inputs copied in between (eager work and synchronisations between the
replays); every replay must match the oracle on those inputs.  A call made
while its stream is captured never splits K, so it allocates nothing."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from harness import inputs
from tests.parity import bf16_bits, bits_to_f64, check_close, dev, say, sentinel_bf16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dg():
    import moe_grouped_gemm_x128_amd as m
    return m


def capture(fn):
    """Warm up `fn` on a side stream, then capture it into a graph."""
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        fn()
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=s):
            fn()
    torch.cuda.synchronize()
    return g


def test_quantiser_graph_replays(dg):
    say("quantiser under graph capture")
    m, k, t, f = 300, 1024, 256, 520
    xa = torch.empty((m, k), dtype=torch.float32, device="cuda")
    xt = torch.empty((t, f), dtype=torch.float32, device="cuda")
    qa = torch.empty((m, k), dtype=torch.uint8, device="cuda")
    sa = torch.empty((m, k // 128), dtype=torch.float32, device="cuda")
    qb = torch.empty((m, k), dtype=torch.uint8, device="cuda")
    sb = torch.empty(((m + 127) // 128, k // 128), dtype=torch.float32, device="cuda")
    qt = torch.empty((f, t), dtype=torch.uint8, device="cuda")
    st = torch.empty((f, t // 128), dtype=torch.float32, device="cuda")

    def work():
        dg.dg_quantize_fp8_1x128(xa, qa, sa)
        dg.dg_quantize_fp8_128x128(xa, qb, sb)
        dg.dg_quantize_fp8_1x128_transposed(xt, qt, st)

    rng = np.random.default_rng(71)
    xa.copy_(torch.from_numpy(rng.standard_normal((m, k), dtype=np.float32)))
    xt.copy_(torch.from_numpy(rng.standard_normal((t, f), dtype=np.float32)))
    g = capture(work)
    for rep in range(3):
        a = (rng.standard_normal((m, k)) * 2.0 ** rng.integers(-8, 8)).astype(np.float32)
        x2 = (rng.standard_normal((t, f)) * 2.0 ** rng.integers(-8, 8)).astype(np.float32)
        xa.copy_(torch.from_numpy(a))
        xt.copy_(torch.from_numpy(x2))
        for o in (qa, qb, qt):
            o.fill_(0x7F)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for (q, s), (qr, sr), what in (((qa, sa), oracle.quantize_1x128(a), "1x128"),
                                       ((qb, sb), oracle.quantize_128x128(a), "128x128"),
                                       ((qt, st), oracle.quantize_1x128_transposed(x2), "transposed")):
            assert np.array_equal(q.cpu().numpy(), qr), f"replay {rep}: {what} codes"
            assert np.array_equal(s.cpu().numpy().view(np.uint32), sr.view(np.uint32)), f"replay {rep}: {what} scales"


@pytest.mark.parametrize("which", ["ue8m0", "bf16"])
def test_gemm_variants_graph_replays(dg, which):
    """Small M (eager calls split K) captured without a split; every replay
    with new operands matches the oracle."""
    m, n, k = 64, 2112, 7168
    say(f"{which} 64x2112x7168 under graph capture")
    kind = dg.KIND_DENSE_POW2 if which == "ue8m0" else dg.KIND_BF16
    assert dg.select_config(kind, m, n, k)["k_splits"] > 1  # eager calls split K; captured ones do not
    if which == "ue8m0":
        d = inputs.make_dense(m, n, k, seed=inputs.SEED_BASE + 72, pow2=True)
        a, sa, b, sb = dev(d.a), dev(d.sa), dev(d.b), dev(d.sb)
        fn = lambda: dg.dg_gemm_fp8_nt_ue8m0(a, sa, b, sb, out)
    else:
        d = inputs.make_dense_bf16(m, n, k, seed=inputs.SEED_BASE + 72)
        to = lambda bits: torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)
        a, b = to(d.a), to(d.b)
        fn = lambda: dg.dg_gemm_bf16_nt(a, b, out)
    out = sentinel_bf16((m, n))
    g = capture(fn)
    for rep in range(3):
        seed = inputs.SEED_BASE + 73 + rep
        if which == "ue8m0":
            e = inputs.make_dense(m, n, k, seed=seed, pow2=True)
            for t, h in ((a, e.a), (sa, e.sa), (b, e.b), (sb, e.sb)):
                t.copy_(dev(h))
            ref, _ = oracle.gemm_fp8_nt(e.a, e.sa, e.b, e.sb)
        else:
            e = inputs.make_dense_bf16(m, n, k, seed=seed)
            a.copy_(to(e.a))
            b.copy_(to(e.b))
            ref, _ = oracle.gemm_bf16_nt(e.a, e.b)
        out.view(torch.int16).fill_(-1)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        check_close(bits_to_f64(bf16_bits(out)), bits_to_f64(ref), f"{which} graph replay {rep}")


def test_quantise_then_gemm_pipeline_graph(dg):
    """fp32 activations and weights -> quantiser -> dense FP8 GEMM, captured as
    one graph; each replay on new fp32 inputs matches the oracle's quantiser
    followed by the oracle GEMM."""
    m, n, k = 256, 640, 1536
    say("quantise -> GEMM pipeline under graph capture")
    xa = torch.empty((m, k), dtype=torch.float32, device="cuda")
    xb = torch.empty((n, k), dtype=torch.float32, device="cuda")
    qa = torch.empty((m, k), dtype=torch.uint8, device="cuda")
    sa = torch.empty((m, k // 128), dtype=torch.float32, device="cuda")
    qb = torch.empty((n, k), dtype=torch.uint8, device="cuda")
    sb = torch.empty(((n + 127) // 128, k // 128), dtype=torch.float32, device="cuda")
    out = sentinel_bf16((m, n))

    def work():
        dg.dg_quantize_fp8_1x128(xa, qa, sa)
        dg.dg_quantize_fp8_128x128(xb, qb, sb)
        dg.dg_gemm_fp8_nt(qa, sa, qb, sb, out)

    rng = np.random.default_rng(74)
    xa.copy_(torch.from_numpy(rng.standard_normal((m, k), dtype=np.float32)))
    xb.copy_(torch.from_numpy(rng.standard_normal((n, k), dtype=np.float32)))
    g = capture(work)
    for rep in range(3):
        a = rng.standard_normal((m, k), dtype=np.float32)
        b = rng.standard_normal((n, k), dtype=np.float32)
        xa.copy_(torch.from_numpy(a))
        xb.copy_(torch.from_numpy(b))
        out.view(torch.int16).fill_(-1)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        oa, osa = oracle.quantize_1x128(a)
        ob, osb = oracle.quantize_128x128(b)
        ref, _ = oracle.gemm_fp8_nt(oa, osa, ob, osb)
        check_close(bits_to_f64(bf16_bits(out)), bits_to_f64(ref), f"pipeline replay {rep}")


def _masked_sample_check(x, bits, what, count=1536):
    """Sampled valid outputs against the oracle; every row past masked_m keeps
    its sentinel bits and every valid row is written."""
    rng = np.random.default_rng(11)
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
        assert np.all(bits[g, valid[g]:] == 0xFFFF), f"{what}: group {g}: rows past masked_m written"
        assert not np.any(bits[g, :valid[g]] == 0xFFFF), f"{what}: group {g}: valid rows left unwritten"


@pytest.mark.parametrize("g,n,k", [(1, 4096, 7168), (1, 7168, 2048), (4, 4096, 7168), (4, 7168, 2048),
                                   (16, 4096, 7168), (16, 7168, 2048)])
def test_masked_graph_replays(dg, g, n, k):
    """The masked decode GEMM captured at the decode workload sizes (the
    pages' graph-captured case): replays with A, its scales and masked_m
    rewritten on the device between them -- including 0, 1, M_max and more
    than M_max rows -- each match the oracle, with the sentinel rows intact."""
    m_max = 256
    x = inputs.make_masked(g, m_max, n, k, seed=inputs.SEED_BASE + 120 + g)
    cfg = dg.select_config(dg.KIND_MASKED, m_max, n, k, g)
    say(f"masked graph G={g} N={n} K={k} (eager plan {cfg})")
    a, sa = dev(x.a).view(torch.float8_e4m3fn), dev(x.sa)
    b, sb = dev(x.b).view(torch.float8_e4m3fn), dev(x.sb)
    mm = dev(x.masked_m)
    out = sentinel_bf16((g, m_max, n))
    graph = capture(lambda: dg.dg_grouped_fp8_masked(a, sa, b, sb, out, mm))
    edge = [0, 1, m_max, m_max + 44]
    rng = np.random.default_rng(g * 7 + k)
    plans = [[edge[i % 4] for i in range(g)],
             list(rng.integers(64, 193, g)),
             [edge[(i + 2) % 4] for i in range(g)]]
    for rep, counts in enumerate(plans):
        y = inputs.make_masked(g, m_max, n, k, seed=inputs.SEED_BASE + 130 + rep, masked_m=counts)
        a.copy_(dev(y.a).view(torch.float8_e4m3fn))
        sa.copy_(dev(y.sa))
        mm.copy_(dev(y.masked_m))
        out.view(torch.int16).fill_(-1)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        y.b, y.sb = x.b, x.sb  # B is not rewritten
        _masked_sample_check(y, bf16_bits(out), f"masked G={g} N={n} K={k} replay {rep} masked_m={counts[:4]}")


def test_contiguous_graph_replays(dg):
    """The contiguous grouped GEMM captured once; replays with m_indices and A
    rewritten on the device: padded segments, an empty expert, a segment
    boundary inside a 256-row tile (two experts in one tile) and stray
    out-of-range ids.  Each replay matches the oracle on every output, padding
    rows keep their sentinel bits."""
    g, rpe, n, k = 4, 512, 640, 2048
    x = inputs.make_contiguous(g, rpe, n, k, seed=inputs.SEED_BASE + 140)
    mt = x.m_total
    say(f"contiguous graph G={g} rows/expert={rpe} N={n} K={k} ({dg.select_config(dg.KIND_CONTIGUOUS, mt, n, k, g)})")
    a, sa = dev(x.a).view(torch.float8_e4m3fn), dev(x.sa)
    b, sb = dev(x.b).view(torch.float8_e4m3fn), dev(x.sb)
    ids = dev(x.m_indices)
    out = sentinel_bf16((mt, n))
    graph = capture(lambda: dg.dg_grouped_fp8_contiguous(a, sa, b, sb, out, ids))

    def layout(kind):
        m = np.full(mt, -1, np.int32)
        if kind == 0:    # the harness's padded segments
            return x.m_indices.copy()
        if kind == 1:    # expert 1 empty; expert 2 takes two segments; 128-row segments
            m[0:384] = 0
            m[512:640] = 2
            m[640:1000] = 2
            m[1024:1100] = 3
            m[1536:1920] = 3
            return m
        # segment boundaries at odd 128-row blocks (a 256-row tile holding two
        # experts), padding at block ends, and out-of-range ids (skipped)
        m[0:128] = 3
        m[128:250] = 0
        m[256:384] = 1
        m[384:500] = 2
        m[640:768] = 7
        m[768:896] = -5
        m[896:1020] = 1
        return m

    for rep in range(3):
        y = inputs.make_contiguous(g, rpe, n, k, seed=inputs.SEED_BASE + 141 + rep)
        mi = layout(rep)
        a.copy_(dev(y.a).view(torch.float8_e4m3fn))
        sa.copy_(dev(y.sa))
        ids.copy_(dev(mi))
        out.view(torch.int16).fill_(-1)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        init = np.full((mt, n), 0xFFFF, np.uint16)
        ref = oracle.grouped_contiguous(y.a, y.sa, x.b, x.sb, mi, init)
        ref_bits = ref[0] if isinstance(ref, tuple) else ref
        got = bf16_bits(out)
        valid = (mi >= 0) & (mi < g)
        assert np.all(got[~valid] == 0xFFFF), f"replay {rep}: padding or out-of-range rows written"
        check_close(bits_to_f64(got[valid]), bits_to_f64(ref_bits[valid]), f"contiguous replay {rep}")


def test_fused_swiglu_graph_replays(dg):
    """The contiguous GEMM with the fused SwiGLU + re-quantise epilogue,
    captured once and replayed with A and m_indices rewritten on the device
    (exact-output operands): every replay gives the oracle composition's codes
    and scales on the valid rows (the stand-alone step's bar) and leaves the
    padding rows' sentinels."""
    g, rpe, i, k = 3, 384, 256, 512
    x = inputs.make_contiguous_exact(g, rpe, 2 * i, k, seed=inputs.SEED_BASE + 150)
    mt = x.m_total
    say(f"fused swiglu graph G={g} rows/expert={rpe} I={i} K={k}")
    a, sa = dev(x.a), dev(x.sa)
    b, sb = dev(x.b), dev(x.sb)
    ids = dev(x.m_indices)
    q = torch.full((mt, i), 0x7F, dtype=torch.uint8, device="cuda")
    s = torch.full((mt, i // 128), float("nan"), dtype=torch.float32, device="cuda")
    graph = capture(lambda: dg.dg_grouped_fp8_contiguous_swiglu(a, sa, b, sb, q, s, ids))
    margin = 2.0 ** -18
    for rep in range(3):
        y = inputs.make_contiguous_exact(g, rpe, 2 * i, k, seed=inputs.SEED_BASE + 151 + rep)
        mi = y.m_indices.copy()
        if rep == 1:
            mi[rpe:2 * rpe] = -1       # an empty expert
        if rep == 2:
            mi[:128] = g + 2           # out-of-range ids are skipped
        a.copy_(dev(y.a))
        sa.copy_(dev(y.sa))
        ids.copy_(dev(mi))
        q.fill_(0x7F)
        s.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got_q, got_s = q.cpu().numpy(), s.cpu().numpy()
        valid = (mi >= 0) & (mi < g)
        assert np.all(got_q[~valid] == 0x7F) and np.all(np.isnan(got_s[~valid])), f"replay {rep}: padding written"
        bits, exact = oracle.grouped_contiguous(y.a, y.sa, x.b, x.sb, mi, np.zeros((mt, 2 * i), np.uint16))
        assert np.array_equal(exact[valid].astype(np.float32).astype(np.float64), exact[valid])
        q_ref, s_ref, h = oracle.swiglu_quantize_1x128(np.ascontiguousarray(bits[valid]))
        gq, gs = got_q[valid], got_s[valid]
        assert np.all(np.abs(gs.astype(np.float64) - s_ref) <= 2.0 ** -20 * s_ref), f"replay {rep}: scales"
        yv = np.clip(h / np.repeat(s_ref.astype(np.float64), 128, axis=1), -448.0, 448.0)
        lo = oracle.e4m3_encode(np.clip(yv * (1 - margin), -448.0, 448.0).astype(np.float32))
        hi = oracle.e4m3_encode(np.clip(yv * (1 + margin), -448.0, 448.0).astype(np.float32))
        firm = lo == hi
        assert np.array_equal(gq[firm], q_ref[firm]), f"replay {rep}: codes"
        assert np.all((gq[~firm] == lo[~firm]) | (gq[~firm] == hi[~firm])), f"replay {rep}: code outside the bracket"
