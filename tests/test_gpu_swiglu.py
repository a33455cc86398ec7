"""GPU parity of dg_swiglu_quantize_fp8_1x128 (SwiGLU on the first linear's
bf16 output, then the 1x128 FP8 quantise) against the CPU oracle.

The activation goes through the exponential, which neither side evaluates
exactly, so the bar is stated on the oracle's exact values: every scale within
2^-20 (relative) of the oracle's, and every code equal to the oracle's except
where the oracle's exact quotient h / s lies within 2^-18 (relative) of the
midpoint between two e4m3 values; there the code must be one of the two, and
such elements must be rare (< 1e-3) on random inputs.  The GPU's h is within a few fp32 ulp of
exact for every gate (the exponential's argument is exact), far inside that margin."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from tests.parity import say

pytestmark = pytest.mark.gpu

MARGIN = 2.0 ** -18


@pytest.fixture(scope="module")
def dg():
    import moe_grouped_gemm_x128_amd as m
    return m


def bf16_bits(x: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16).view(torch.int16) \
        .numpy().view(np.uint16)


def linear1_output(seed, m, i, lo=-3, hi=2):
    """bf16 bits [m, 2i] shaped like a GEMM output: N(0,1) times 2^U(lo, hi)
    per row (|gate| stays below 32)."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((m, 2 * i), dtype=np.float32) * np.float32(2.0) ** rng.integers(lo, hi, (m, 1))
    return bf16_bits(x.astype(np.float32))


def to_dev(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def run(dg, c_bits):
    m, i2 = c_bits.shape
    i = i2 // 2
    q = torch.full((m, i), 0x7F, dtype=torch.uint8, device="cuda")   # NaN code: unwritten outputs show
    s = torch.full((m, i // 128), float("nan"), dtype=torch.float32, device="cuda")
    dg.dg_swiglu_quantize_fp8_1x128(to_dev(c_bits), q, s)
    torch.cuda.synchronize()
    return q.cpu().numpy(), s.cpu().numpy()


def check(q, s, c_bits, what, rare=True):
    q_ref, s_ref, h = oracle.swiglu_quantize_1x128(c_bits)
    assert np.all(np.abs(s.astype(np.float64) - s_ref) <= 2.0 ** -20 * s_ref), f"{what}: scales"
    y = np.clip(h / np.repeat(s_ref.astype(np.float64), 128, axis=1), -448.0, 448.0)
    lo = oracle.e4m3_encode(np.clip(y * (1 - MARGIN), -448.0, 448.0).astype(np.float32))
    hi = oracle.e4m3_encode(np.clip(y * (1 + MARGIN), -448.0, 448.0).astype(np.float32))
    firm = lo == hi
    assert np.array_equal(q[firm], q_ref[firm]), \
        f"{what}: {int(np.count_nonzero(q[firm] != q_ref[firm]))} codes differ away from a midpoint"
    loose = ~firm
    assert np.all((q[loose] == lo[loose]) | (q[loose] == hi[loose])), f"{what}: code outside the bracket"
    assert not rare or loose.mean() < 1e-3, f"{what}: {loose.mean():.2e} of the elements near a midpoint"


@pytest.mark.parametrize("m,i", [(1, 128), (3, 384), (17, 128), (300, 2048), (129, 3584), (64, 640)])
def test_swiglu_quant_ragged(dg, m, i):
    say(f"swiglu quantise {m}x{2 * i}")
    c = linear1_output(100 + m + i, m, i)
    q, s = run(dg, c)
    check(q, s, c, f"{m}x{2 * i}")
    q2, s2 = run(dg, c)
    assert np.array_equal(q, q2) and np.array_equal(s.view(np.uint32), s2.view(np.uint32)), "not deterministic"


def test_swiglu_quant_special_rows(dg):
    """Zero gate or up halves (a zero group: codes +-0 with the sign of h,
    scale 1), saturated gates (+-100: silu = gate, and silu = -0), tiny
    products (scale below 2^-60) and large ones (2^100), and gates in
    [-80, -20] (h = gate * e^gate * up down to 1e-33, where a rounded
    exponential argument would cost |gate| * 2^-24 of relative error)."""
    i = 256
    rng = np.random.default_rng(7)
    rows = []
    g, u = rng.standard_normal(i), rng.standard_normal(i)
    rows.append(np.concatenate([np.zeros(i), u]))
    rows.append(np.concatenate([g, np.zeros(i)]))
    rows.append(np.concatenate([np.where(rng.random(i) < 0.5, 100.0, -100.0), u]))
    rows.append(np.concatenate([g, u * 2.0 ** -110]))
    rows.append(np.concatenate([g, u * 2.0 ** 100]))
    rows.append(np.concatenate([np.concatenate([g[:128] * 8, g[128:] / 8]), u]))
    rows.append(np.concatenate([-20.0 - 60.0 * rng.random(i), u]))
    c = bf16_bits(np.stack(rows).astype(np.float32))
    say("swiglu quantise special rows")
    q, s = run(dg, c)
    check(q, s, c, "special rows", rare=False)  # gate = 100 rows put h / s on exact midpoints
    assert np.all(s[:2] == 1.0) and np.all((q[:2] & 0x7F) == 0)


@pytest.mark.parametrize("m,i", [(65536, 2048), (16 * 256, 3584)])
def test_swiglu_quant_full_size(dg, m, i):
    """The first linear's output at full size: G=8 experts x 8192 rows with
    N = 2I = 4096, and a masked decode batch (16 groups x 256 rows) with
    N = 7168; every output compared."""
    say(f"swiglu quantise full {m}x{2 * i}")
    c = linear1_output(5, m, i)
    q, s = run(dg, c)
    check(q, s, c, f"full {m}x{2 * i}")


def test_swiglu_quant_graph_replays(dg):
    """Captured once, replayed with new inputs copied in between."""
    m, i = 200, 1024
    say("swiglu quantise under graph capture")
    c = to_dev(linear1_output(11, m, i))
    q = torch.empty((m, i), dtype=torch.uint8, device="cuda")
    s = torch.empty((m, i // 128), dtype=torch.float32, device="cuda")
    st = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(st):
        dg.dg_swiglu_quantize_fp8_1x128(c, q, s)
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=st):
            dg.dg_swiglu_quantize_fp8_1x128(c, q, s)
    torch.cuda.synchronize()
    for rep in range(3):
        bits = linear1_output(12 + rep, m, i)
        c.copy_(to_dev(bits))
        q.fill_(0x7F)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        check(q.cpu().numpy(), s.cpu().numpy(), bits, f"graph replay {rep}")


def test_swiglu_then_gemm(dg):
    """The re-quantised activation feeds the second GEMM: the GPU's
    swiglu-quantise then the GPU dense GEMM, against the oracle's
    swiglu-quantise then the oracle GEMM (a code that differs at a midpoint
    moves one product by one e4m3 step, far inside the GEMM's bar)."""
    from harness import inputs
    from tests.parity import bf16_bits as out_bits, bits_to_f64, check_close, dev, sentinel_bf16
    m, i, n = 256, 1024, 384
    say("swiglu quantise -> GEMM")
    c = linear1_output(21, m, i)
    q, s = run(dg, c)
    q_ref, s_ref, _ = oracle.swiglu_quantize_1x128(c)
    w = inputs.make_dense(8, n, i, seed=inputs.SEED_BASE + 90)   # weights B [n, i] with 128x128 scales
    out = sentinel_bf16((m, n))
    dg.dg_gemm_fp8_nt(dev(q), dev(s), dev(w.b), dev(w.sb), out)
    torch.cuda.synchronize()
    ref, _ = oracle.gemm_fp8_nt(q_ref, s_ref, w.b, w.sb)
    check_close(bits_to_f64(out_bits(out)), bits_to_f64(ref), "swiglu -> GEMM")
