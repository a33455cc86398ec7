"""The entry points added beside the GEMM family under HIP graph capture:
the quantiser, the power-of-two-scale GEMM and the BF16 GEMM, alone and as
one captured quantise -> GEMM pipeline.  Each graph is replayed several times
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
