"""GPU parity of the FP8 quantiser against the CPU oracle: codes and scales
must match bit for bit (integer work decided in fp32 on both sides), on
every output, at small ragged shapes and at the operand sizes of the GEMM
workloads.  Outputs are prefilled with a pattern the quantiser never writes
(code 0x7F is NaN, scales NaN), so an element left unwritten fails."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from tests.parity import say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dg():
    import moe_grouped_gemm_x128_amd as m
    return m


def data(seed, rows, cols, group_axis=1):
    """N(0,1) fp32 (the workloads' input distribution) with a different
    binade per 128-element group along `group_axis`, a few all-zero groups
    and some negative zeros, so scales, subnormal codes and ties all occur."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((rows, cols)).astype(np.float32)
    if group_axis == 1 and cols % 128 == 0:
        mag = (2.0 ** rng.integers(-10, 10, size=(rows, cols // 128))).astype(np.float32)
        x = (x.reshape(rows, -1, 128) * mag[:, :, None]).reshape(rows, cols)
    elif group_axis == 0 and rows % 128 == 0:
        mag = (2.0 ** rng.integers(-10, 10, size=(rows // 128, cols))).astype(np.float32)
        x = (x.reshape(-1, 128, cols) * mag[:, None, :]).reshape(rows, cols)
    if rows > 3 and cols > 3:
        if group_axis == 1:
            x[rows // 2, : min(cols, 128)] = 0.0
        else:
            x[: min(rows, 128), cols // 2] = 0.0
        x[:, cols // 3] *= np.float32(2.0 ** -12)
        x[0, 1] = -0.0
    return np.ascontiguousarray(x)


def run(fn, x, qshape, sshape):
    xd = torch.from_numpy(x).cuda()
    q = torch.full(qshape, 0x7F, dtype=torch.uint8, device="cuda")
    s = torch.full(sshape, float("nan"), dtype=torch.float32, device="cuda")
    fn(xd, q, s)
    torch.cuda.synchronize()
    return q.cpu().numpy(), s.cpu().numpy()


def check(got, ref, what):
    (q, s), (qr, sr) = got, ref
    assert q.shape == qr.shape and s.shape == sr.shape, what
    bad = np.flatnonzero(q != qr)
    assert bad.size == 0, f"{what}: {bad.size} codes differ, first at {np.unravel_index(bad[0], q.shape)}: " \
                          f"gpu {q.flat[bad[0]]:#04x} oracle {qr.flat[bad[0]]:#04x}"
    assert np.array_equal(s.view(np.uint32), sr.view(np.uint32)), f"{what}: scales differ"


@pytest.mark.parametrize("m,k", [(1, 128), (37, 384), (128, 256), (130, 640), (300, 1024), (257, 7168)])
def test_1x128_small(dg, m, k):
    say(f"quantize 1x128 {m}x{k}")
    x = data(m * 7 + k, m, k)
    got = run(dg.dg_quantize_fp8_1x128, x, (m, k), (m, k // 128))
    check(got, oracle.quantize_1x128(x), f"1x128 {m}x{k}")
    assert all(np.array_equal(a, b) for a, b in zip(got, run(dg.dg_quantize_fp8_1x128, x, (m, k), (m, k // 128)))), \
        "not deterministic"


@pytest.mark.parametrize("n,k", [(1, 128), (100, 256), (128, 128), (300, 384), (2112, 512)])
def test_128x128_small(dg, n, k):
    say(f"quantize 128x128 {n}x{k}")
    x = data(n * 5 + k, n, k)
    if k >= 256:
        x[: min(n, 128), 128:256] = 0.0  # an all-zero block: scale 1, codes 0
    nb = (n + 127) // 128
    got = run(dg.dg_quantize_fp8_128x128, x, (n, k), (nb, k // 128))
    check(got, oracle.quantize_128x128(x), f"128x128 {n}x{k}")


@pytest.mark.parametrize("t,f", [(128, 4), (128, 200), (384, 260), (256, 128), (1024, 516)])
def test_1x128_transposed_small(dg, t, f):
    say(f"quantize 1x128 transposed {t}x{f}")
    x = data(t * 3 + f, t, f, group_axis=0)
    got = run(dg.dg_quantize_fp8_1x128_transposed, x, (f, t), (f, t // 128))
    check(got, oracle.quantize_1x128_transposed(x), f"transposed {t}x{f}")


@pytest.mark.parametrize("mode", ["1x128", "128x128", "transposed"])
def test_extreme_magnitudes(dg, mode):
    """Group maxima from 2^-130 to 2^120 (scales below 2^-60 take the
    quotient's rescaled path), fp32 subnormal inputs inside normal groups,
    negative zeros: still bit-exact."""
    say(f"quantize extreme magnitudes {mode}")
    rng = np.random.default_rng(4242)
    rows, cols = 256, 1024
    x = rng.standard_normal((rows, cols)).astype(np.float64)
    if mode == "transposed":
        e = rng.integers(-130, 120, size=(rows // 128, cols))
        x = x * np.repeat(2.0 ** e, 128, axis=0)
    else:
        e = rng.integers(-130, 120, size=(rows, cols // 128))
        x = x * np.repeat(2.0 ** e, 128, axis=1)
    x = x.astype(np.float32)
    x[5, 3:40] = np.float32(1e-41)       # subnormal values in a normal group
    x[7, 9] = np.float32(-0.0)
    amax = np.abs(x).max()
    assert np.isfinite(amax)
    if mode == "1x128":
        got = run(dg.dg_quantize_fp8_1x128, x, (rows, cols), (rows, cols // 128))
        ref = oracle.quantize_1x128(x)
    elif mode == "128x128":
        got = run(dg.dg_quantize_fp8_128x128, x, (rows, cols), (rows // 128, cols // 128))
        ref = oracle.quantize_128x128(x)
    else:
        got = run(dg.dg_quantize_fp8_1x128_transposed, x, (cols, rows), (cols, rows // 128))
        ref = oracle.quantize_1x128_transposed(x)
    check(got, ref, f"extreme magnitudes {mode}")


@pytest.mark.parametrize("what,rows,cols", [
    ("activations 1x128", 4096, 7168),     # the pages' usage example LHS, [4096, 7168] with [4096, 56] scales
    ("weights 128x128", 2112, 7168),       # its RHS, [2112, 7168] with [17, 56] scales
    ("weights 128x128", 7168, 16384),      # the largest dense-sweep weight
    ("tokens transposed", 4096, 7168),     # weight-gradient operand: X [4096 tokens, 7168] -> [7168, 4096]
])
def test_full_size(dg, what, rows, cols):
    """Workload-size operands, every output compared."""
    say(f"quantize {what} {rows}x{cols}")
    rng = np.random.default_rng(rows + cols)
    x = rng.standard_normal((rows, cols), dtype=np.float32)
    if what.startswith("activations"):
        got = run(dg.dg_quantize_fp8_1x128, x, (rows, cols), (rows, cols // 128))
        ref = oracle.quantize_1x128(x)
    elif what.startswith("weights"):
        got = run(dg.dg_quantize_fp8_128x128, x, (rows, cols), ((rows + 127) // 128, cols // 128))
        ref = oracle.quantize_128x128(x)
    else:
        got = run(dg.dg_quantize_fp8_1x128_transposed, x, (cols, rows), (cols, rows // 128))
        ref = oracle.quantize_1x128_transposed(x)
    check(got, ref, f"{what} {rows}x{cols}")


def test_quantised_operands_feed_the_gemm(dg):
    """End to end on the GPU: quantise fp32 activations and weights, run the
    dense GEMM on them, and compare with the oracle GEMM of the oracle's own
    quantisation of the same fp32 inputs (identical bytes, so the GEMM bar)."""
    from tests.parity import bf16_bits, bits_to_f64, check_close
    m, n, k = 256, 384, 1024
    rng = np.random.default_rng(99)
    a32 = rng.standard_normal((m, k), dtype=np.float32)
    b32 = rng.standard_normal((n, k), dtype=np.float32)
    qa, sa = dg.quantize_fp8_1x128(torch.from_numpy(a32).cuda())
    qb, sb = dg.quantize_fp8_128x128(torch.from_numpy(b32).cuda())
    c = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
    dg.dg_gemm_fp8_nt(qa, sa, qb, sb, c)
    torch.cuda.synchronize()
    oa, osa = oracle.quantize_1x128(a32)
    ob, osb = oracle.quantize_128x128(b32)
    assert np.array_equal(qa.view(torch.uint8).cpu().numpy(), oa)
    assert np.array_equal(qb.view(torch.uint8).cpu().numpy(), ob)
    ref, _ = oracle.gemm_fp8_nt(oa, osa, ob, osb)
    check_close(bits_to_f64(bf16_bits(c)), bits_to_f64(ref),
                "quantise + dense GEMM 256x384x1024")


# ---- power-of-two (UE8M0) scales, packed four to an int32 -------------------

def run_ue8m0(fn, x, qshape, sshape):
    """Codes prefilled with 0x7F (NaN) and words with 0x7F7F7F7F, which no
    group writes (its E is at most 254 and padding bytes are 0)."""
    xd = torch.from_numpy(x).cuda()
    q = torch.full(qshape, 0x7F, dtype=torch.uint8, device="cuda")
    s = torch.full(sshape, 0x7F7F7F7F, dtype=torch.int32, device="cuda")
    fn(xd, q, s)
    torch.cuda.synchronize()
    return q.cpu().numpy(), s.cpu().numpy()


def check_ue8m0(got, ref, what):
    (q, s), (qr, sr) = got, ref
    assert q.shape == qr.shape and s.shape == sr.shape, what
    bad = np.flatnonzero(q != qr)
    assert bad.size == 0, f"{what}: {bad.size} codes differ, first at {np.unravel_index(bad[0], q.shape)}: " \
                          f"gpu {q.flat[bad[0]]:#04x} oracle {qr.flat[bad[0]]:#04x}"
    assert np.array_equal(s, sr), f"{what}: {int(np.count_nonzero(s != sr))} packed scale words differ"


def wide_data(seed, rows, cols):
    """data() with group magnitudes over 2^-130 .. 2^100, so the codes E run
    from 0 (scales below the E8M0 range) to 227 and subnormal scales occur."""
    x = data(seed, rows, cols)
    rng = np.random.default_rng(seed + 1)
    mag = np.ldexp(np.float32(1.0), rng.integers(-130, 100, size=(rows, cols // 128))).astype(np.float32)
    return np.ascontiguousarray((x.reshape(rows, -1, 128) * mag[:, :, None]).reshape(rows, cols).astype(np.float32))


@pytest.mark.parametrize("m,k", [(1, 128), (37, 384), (128, 512), (130, 640), (300, 1152), (257, 7168)])
def test_1x128_ue8m0(dg, m, k):
    """K/128 = 1, 3, 4, 5, 9, 56 groups per row: whole and padded words."""
    say(f"quantize 1x128 ue8m0 {m}x{k}")
    for x in (data(m * 11 + k, m, k), wide_data(m * 13 + k, m, k)):
        got = run_ue8m0(dg.dg_quantize_fp8_1x128_ue8m0, x, (m, k), (m, (k // 128 + 3) // 4))
        check_ue8m0(got, oracle.quantize_1x128_ue8m0(x), f"1x128 ue8m0 {m}x{k}")


@pytest.mark.parametrize("n,k", [(1, 128), (100, 384), (128, 512), (300, 640), (2112, 1152)])
def test_128x128_ue8m0(dg, n, k):
    say(f"quantize 128x128 ue8m0 {n}x{k}")
    x = data(n * 17 + k, n, k)
    if k >= 256:
        x[: min(n, 128), 128:256] = 0.0  # an all-zero block: code 127, codes 0
    nb = (n + 127) // 128
    got = run_ue8m0(dg.dg_quantize_fp8_128x128_ue8m0, x, (n, k), (nb, (k // 128 + 3) // 4))
    check_ue8m0(got, oracle.quantize_128x128_ue8m0(x), f"128x128 ue8m0 {n}x{k}")


def test_ue8m0_quantise_then_packed_gemm(dg):
    """The power-of-two path end to end on the GPU: both operands quantised
    with packed UE8M0 scales, then the packed GEMM, against the oracle's
    quantiser and GEMM on the same fp32 inputs."""
    from tests.parity import bf16_bits, bits_to_f64, check_close, sentinel_bf16
    m, n, k = 300, 520, 1664
    rng = np.random.default_rng(91)
    xa = rng.standard_normal((m, k)).astype(np.float32)
    xb = rng.standard_normal((n, k)).astype(np.float32)
    say("ue8m0 quantise -> packed GEMM")
    qa, sa = dg.quantize_fp8_1x128_ue8m0(torch.from_numpy(xa).cuda())
    qb, sb = dg.quantize_fp8_128x128_ue8m0(torch.from_numpy(xb).cuda())
    c = sentinel_bf16((m, n))
    dg.dg_gemm_fp8_nt_ue8m0_packed(qa, sa, qb, sb, c)
    torch.cuda.synchronize()
    ra, wa = oracle.quantize_1x128_ue8m0(xa)
    rb, wb = oracle.quantize_128x128_ue8m0(xb)
    assert np.array_equal(qa.view(torch.uint8).cpu().numpy(), ra) and np.array_equal(sa.cpu().numpy(), wa)
    assert np.array_equal(qb.view(torch.uint8).cpu().numpy(), rb) and np.array_equal(sb.cpu().numpy(), wb)
    ref, _ = oracle.gemm_fp8_nt_ue8m0_packed(ra, wa, rb, wb)
    check_close(bits_to_f64(bf16_bits(c)), bits_to_f64(ref), "ue8m0 quantise -> GEMM")
