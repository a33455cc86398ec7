"""Pins for the quantiser oracle (oracle/dg_quant_oracle.c), on the CPU.

Each test checks the oracle against something other than itself: torch's
float8_e4m3fn cast (a library routine) on every tie point between e4m3 values
and its fp32 neighbours, a brute-force nearest search over the decoded e4m3
grid, the input harness's numpy + torch quantiser (an independent
implementation of the same rule), and invariants the rule implies (a +-448 code
in every non-zero group, the rounding error bound, exact power-of-two
rescaling, sign symmetry).  Planted mistakes in copies of the oracle must each
fail one of them.
"""
from __future__ import annotations

import os
import subprocess

import numpy as np
import pytest
import torch

import oracle
from harness import inputs
from tests import exact_ref as X

ORACLE_DIR = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle")


def torch_encode(y: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(y, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def finite_grid() -> np.ndarray:
    """Every non-negative finite e4m3 value, ascending (torch's decode)."""
    v = X.torch_decode(np.arange(0, 0x7F, dtype=np.uint8))
    return np.unique(v[np.isfinite(v)])


def tie_points() -> np.ndarray:
    """The grid, every midpoint between neighbours (exact in fp32), the fp32
    neighbours of each, both signs."""
    g = finite_grid().astype(np.float32)
    mid = ((g[:-1].astype(np.float64) + g[1:]) / 2).astype(np.float32)
    pts = np.concatenate([g, mid, np.nextafter(mid, np.float32(np.inf)), np.nextafter(mid, np.float32(0)),
                          np.nextafter(g, np.float32(0)), np.array([2.0 ** -10, 2.0 ** -11, 1e-30], np.float32)])
    pts = pts[(pts >= 0) & (pts <= 448)]
    return np.concatenate([pts, -pts]).astype(np.float32)


def grouped_data(rng, rows, cols, zero_groups=True):
    """N(0,1) fp32 with a different binade per 128-wide group (so scales span
    many magnitudes) and, optionally, some all-zero groups."""
    x = rng.standard_normal((rows, cols)).astype(np.float32)
    mag = (2.0 ** rng.integers(-12, 12, size=(rows, cols // 128))).astype(np.float32)
    x = (x.reshape(rows, cols // 128, 128) * mag[:, :, None]).reshape(rows, cols)
    if zero_groups and rows > 2 and cols >= 256:
        x[1, 128:256] = 0.0
        x[2, :128] = -0.0
    return x


# ---------------------------------------------------------------- pins -----

def pin_encode_ties() -> bool:
    y = tie_points()
    return np.array_equal(oracle.e4m3_encode(y), torch_encode(y))


def pin_encode_random() -> bool:
    rng = np.random.default_rng(11)
    y = (rng.uniform(-1, 1, 200000) * 2.0 ** rng.uniform(-12, 8.8, 200000)).astype(np.float32)
    y = np.clip(y, -448, 448)
    return np.array_equal(oracle.e4m3_encode(y), torch_encode(y))


def pin_encode_brute_force() -> bool:
    """Nearest value of the decoded grid, ties to the even code."""
    rng = np.random.default_rng(12)
    y = (rng.uniform(-1, 1, 3000) * 2.0 ** rng.uniform(-11, 8.8, 3000)).astype(np.float32)
    y = np.concatenate([np.clip(y, -448, 448), tie_points()[::7]]).astype(np.float32)
    codes = np.arange(0, 0x7F, dtype=np.uint8)
    vals = X.torch_decode(codes)
    got = oracle.e4m3_encode(y)
    for yi, gi in zip(y.tolist(), got.tolist()):
        d = np.abs(vals - abs(yi))
        best = np.flatnonzero(d == d.min())
        c = int(codes[best[0]] if len(best) == 1 else [codes[b] for b in best if codes[b] % 2 == 0][0])
        if yi < 0 or (yi == 0 and np.signbit(np.float32(yi))):
            c |= 0x80
        if c != gi:
            return False
    return True


def pin_1x128_vs_harness() -> bool:
    x = grouped_data(np.random.default_rng(13), 37, 640)
    q, s = oracle.quantize_1x128(x)
    qh, sh = inputs.quantize_1x128(x)
    return np.array_equal(q, qh) and np.array_equal(s.view(np.uint32), sh.view(np.uint32))


def pin_128x128_vs_harness() -> bool:
    rng = np.random.default_rng(14)
    x = rng.standard_normal((300, 384)).astype(np.float32) * np.float32(3.0)
    x[128:256, 128:256] *= np.float32(2.0 ** -9)
    x[256:, 256:] = 0.0
    q, s = oracle.quantize_128x128(x)
    qh, sh = inputs.quantize_128x128(x)
    return s.shape == (3, 3) and np.array_equal(q, qh) and np.array_equal(s.view(np.uint32), sh.view(np.uint32))


def pin_transposed_vs_harness() -> bool:
    x = grouped_data(np.random.default_rng(15), 256, 384).T.copy()  # [T=384, F=256]
    x = x[:, :200]
    q, s = oracle.quantize_1x128_transposed(x)
    qh, sh = inputs.quantize_1x128(np.ascontiguousarray(x.T))
    return q.shape == (200, 384) and np.array_equal(q, qh) and np.array_equal(s, sh)


def pin_invariants() -> bool:
    rng = np.random.default_rng(16)
    x = grouped_data(rng, 24, 512)
    q, s = oracle.quantize_1x128(x)
    g = x.reshape(24, 4, 128)
    qg = q.reshape(24, 4, 128)
    ok = True
    nz = np.abs(g).max(axis=2) > 0
    has448 = ((qg & 0x7F) == 0x7E).any(axis=2)
    ok &= bool(np.all(has448[nz])) and bool(np.all(s[~nz] == 1.0)) and bool(np.all((qg[~nz] & 0x7F) == 0))
    # rounding error bound: half a quantum of the e4m3 grid, relative 2^-4 for
    # normals, 2^-10 absolute (times s) in the subnormal range
    deq = X.torch_decode(qg).astype(np.float64) * s[:, :, None].astype(np.float64)
    err = np.abs(deq - g.astype(np.float64))
    bound = 2.0 ** -4 * np.abs(g) + 2.0 ** -10 * s[:, :, None].astype(np.float64) * 1.0000001
    ok &= bool(np.all(err <= bound))
    # power-of-two rescaling is exact; negation flips the sign bit only
    q2, s2 = oracle.quantize_1x128(x * np.float32(2.0 ** 5))
    ok &= np.array_equal(q2, q) and np.array_equal(s2[nz], s[nz] * np.float32(32.0)) and bool(np.all(s2[~nz] == 1.0))
    q3, s3 = oracle.quantize_1x128(-x)
    ok &= np.array_equal(q3, q ^ 0x80) and np.array_equal(s3, s)
    return ok


PINS = {
    "encode_ties": pin_encode_ties,
    "encode_random": pin_encode_random,
    "encode_brute_force": pin_encode_brute_force,
    "1x128_vs_harness": pin_1x128_vs_harness,
    "128x128_vs_harness": pin_128x128_vs_harness,
    "transposed_vs_harness": pin_transposed_vs_harness,
    "invariants": pin_invariants,
}


@pytest.mark.parametrize("name", sorted(PINS))
def test_quantiser_oracle_pin(name):
    assert PINS[name](), name


def test_encode_round_trips_every_finite_code():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    assert np.array_equal(oracle.e4m3_encode(X.torch_decode(codes).astype(np.float32)), codes)


def test_page_shapes_of_the_scale_tensors():
    """The usage example pairs M=4096, N=2112, K=7168 with [4096, 56] and
    [17, 56] scale tensors: the quantiser's outputs have those shapes."""
    rng = np.random.default_rng(17)
    _, sa = oracle.quantize_1x128(rng.standard_normal((8, 7168)).astype(np.float32))
    _, sb = oracle.quantize_128x128(rng.standard_normal((2112, 256)).astype(np.float32))
    assert sa.shape == (8, 56) and sb.shape == (17, 2)


# ------------------------------------------------------- planted mistakes ---

MUTATIONS = {
    "truncating_round": ("double n = nearbyint(ldexp(a, 3 - E));", "double n = floor(ldexp(a, 3 - E));"),
    "ties_away_from_zero": ("double n = nearbyint(ldexp(a, 3 - E));", "double n = round(ldexp(a, 3 - E));"),
    "subnormal_quantum": ("const double n = nearbyint(ldexp(a, 9));", "const double n = nearbyint(ldexp(a, 10));"),
    "exponent_bias_8": ("((unsigned)(E + 7) << 3)", "((unsigned)(E + 8) << 3)"),
    "fnuz_largest": ("#define E4M3_LARGEST 448.0f", "#define E4M3_LARGEST 240.0f"),
    "group_of_64": ("for (int i = 0; i < QG; ++i) amax = fmaxf(amax, fabsf(xg[i]));",
                    "for (int i = 0; i < 64; ++i) amax = fmaxf(amax, fabsf(xg[i]));"),
    "block_first_row_only": ("for (int64_t r = r0; r < r1; ++r)\n        for (int i = 0; i < QG; ++i) amax",
                             "for (int64_t r = r0; r < r0 + 1; ++r)\n        for (int i = 0; i < QG; ++i) amax"),
    "zero_group_scale_zero": ("return amax == 0.0f ? 1.0f : amax / E4M3_LARGEST;", "return amax / E4M3_LARGEST;"),
    "transpose_index_swapped": ("xt[j * t + i] = x[i * f + j];", "xt[i * f + j] = x[i * f + j];"),
}


def test_real_quantiser_passes_every_pin():
    assert [n for n, f in PINS.items() if not f()] == []


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_quantiser_mistake_is_caught(name, tmp_path):
    old, new = MUTATIONS[name]
    src = open(os.path.join(ORACLE_DIR, "dg_quant_oracle.c")).read()
    assert src.count(old) == 1, f"mutation anchor for {name} not found"
    (tmp_path / "q.c").write_text(src.replace(old, new))
    so = tmp_path / "libmut.so"
    subprocess.run(["gcc", "-O1", "-ffp-contract=off", "-fopenmp", "-shared", "-fPIC", "-o", str(so),
                    os.path.join(ORACLE_DIR, "dg_oracle.c"), str(tmp_path / "q.c"), "-lm"], check=True)
    with oracle.using_library(str(so)):
        failed = []
        for n, f in PINS.items():
            try:
                ok = f()
            except Exception:
                ok = False
            if not ok:
                failed.append(n)
    assert failed, f"planted mistake {name} was not caught by any pin"
