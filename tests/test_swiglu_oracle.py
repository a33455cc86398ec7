"""Pins for the SwiGLU + 1x128 quantise oracle (dgo_swiglu_quantize_1x128 in
oracle/dg_quant_oracle.c), on the CPU.

Each pin checks the oracle against something other than itself: scipy's
logistic function (a library routine) for the activation, the input harness's
numpy + torch quantiser (an independent implementation of the 1x128 rule) for
the composition, a pure-Python brute force (math.exp, a nearest search over
the decoded e4m3 grid) on tiny inputs, and closed forms of silu.  Planted
mistakes in copies of the oracle must each fail one of them.
"""
from __future__ import annotations

import math
import os
import subprocess

import numpy as np
import pytest
import torch
from scipy.special import expit

import oracle
from harness import inputs
from tests import exact_ref as X

ORACLE_DIR = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle")


def bf16_bits(x: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16).view(torch.int16) \
        .numpy().view(np.uint16)


def bf16_value(bits: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(bits, np.uint16).view(np.int16)).view(torch.bfloat16) \
        .to(torch.float64).numpy()


def linear1_output(rng, m, i, lo=-3, hi=2):
    """bf16 [m, 2i] shaped like a GEMM output: N(0,1) times 2^U(lo, hi) per row."""
    x = rng.standard_normal((m, 2 * i)) * 2.0 ** rng.integers(lo, hi, (m, 1))
    return bf16_bits(x.astype(np.float32))


def reference_h(c: np.ndarray) -> np.ndarray:
    """silu(gate) * up in fp64 through scipy's logistic function."""
    i = c.shape[1] // 2
    g, u = bf16_value(c[:, :i]), bf16_value(c[:, i:])
    return g * expit(g) * u


def pin_activation_vs_scipy() -> bool:
    rng = np.random.default_rng(1)
    c = linear1_output(rng, 37, 256)
    _, _, h = oracle.swiglu_quantize_1x128(c)
    ref = reference_h(c)
    return bool(np.all(np.abs(h - ref) <= 4e-16 * np.abs(ref) + 1e-300))


def pin_composition_vs_harness() -> bool:
    """Codes and scales equal the harness quantiser applied to fp32(h), h from
    scipy; groups where scipy's and the oracle's h round to different fp32
    values (last-bit ties) are skipped, and must be rare."""
    rng = np.random.default_rng(2)
    m, i = 64, 512
    c = linear1_output(rng, m, i)
    q, s, h = oracle.swiglu_quantize_1x128(c)
    h32 = reference_h(c).astype(np.float32)
    qr, sr = inputs.quantize_1x128(h32)
    with np.errstate(over="ignore"):
        same = (h.astype(np.float32) == h32).reshape(m, i // 128, 128).all(axis=2)
    if same.mean() < 0.99:
        return False
    qg, qrg = q.reshape(m, i // 128, 128), qr.reshape(m, i // 128, 128)
    return bool(np.array_equal(qg[same], qrg[same]) and np.array_equal(s[same], sr[same]))


def _brute_code(y: float, grid: np.ndarray, codes: np.ndarray) -> int:
    """The e4m3 code nearest to y (|y| <= 448), ties to the even code."""
    a = abs(y)
    d = np.abs(grid - a)
    best = np.flatnonzero(d == d.min())
    code = int(codes[best[0]]) if best.size == 1 else int(min(codes[best], key=lambda v: v & 1))
    return code | (0x80 if math.copysign(1.0, y) < 0 else 0)


def pin_brute_force() -> bool:
    rng = np.random.default_rng(3)
    m, i = 3, 256
    c = linear1_output(rng, m, i)
    c[1, :128] = 0  # a zero gate group: h = +-0, scale 1
    q, s, _ = oracle.swiglu_quantize_1x128(c)
    codes = np.arange(0, 0x7F, dtype=np.uint8)
    grid = X.torch_decode(codes).astype(np.float64)
    for r in range(m):
        for gi in range(i // 128):
            hs = []
            for j in range(gi * 128, gi * 128 + 128):
                g = float(bf16_value(c[r, j]))
                u = float(bf16_value(c[r, i + j]))
                hs.append(np.float32(g / (1.0 + math.exp(-g)) * u))
            amax = max(abs(v) for v in hs)
            sc = np.float32(1.0) if amax == 0 else np.float32(amax) / np.float32(448.0)
            if s[r, gi] != sc:
                return False
            for t, v in enumerate(hs):
                y = float(np.clip(np.float32(v) / sc, -448.0, 448.0))
                if int(q[r, gi * 128 + t]) != _brute_code(y, grid, codes):
                    return False
    return True


def pin_closed_forms() -> bool:
    """silu(x) - silu(-x) = x; silu(0) = 0; silu(x) -> x and -> 0 for large
    |x|; an all-zero up half gives a zero group with scale 1."""
    i = 128
    g = np.linspace(-6.0, 6.0, i).astype(np.float32)
    one = np.ones(i, np.float32)
    c = np.stack([np.concatenate([g, one]), np.concatenate([-g, one]),
                  np.concatenate([np.full(i, 100.0, np.float32), one]),
                  np.concatenate([np.full(i, -100.0, np.float32), one]),
                  np.concatenate([g, np.zeros(i, np.float32)])])
    cb = bf16_bits(c)
    q, s, h = oracle.swiglu_quantize_1x128(cb)
    gv = bf16_value(cb[0, :i])
    ok = bool(np.all(np.abs((h[0] - h[1]) - gv) <= 1e-15 * np.maximum(1.0, np.abs(gv))))
    ok &= bool(h[0, np.flatnonzero(gv == 0)].size == 0 or np.all(h[0, gv == 0] == 0))
    ok &= bool(np.all(h[2] == 100.0)) and bool(np.all(np.abs(h[3]) < 1e-40))
    ok &= bool(s[4, 0] == 1.0) and bool(np.all((q[4] & 0x7F) == 0))
    return ok


PINS = {"activation_vs_scipy": pin_activation_vs_scipy, "composition_vs_harness": pin_composition_vs_harness,
        "brute_force": pin_brute_force, "closed_forms": pin_closed_forms}


@pytest.mark.parametrize("name", sorted(PINS))
def test_swiglu_oracle_pin(name):
    assert PINS[name](), name


MUTATIONS = {
    "exp_sign": ("return x / (1.0 + exp(-x));", "return x / (1.0 + exp(x));"),
    "gate_up_swapped": ("silu(bf16_to_double(gate[j])) * bf16_to_double(up[j])",
                        "silu(bf16_to_double(up[j])) * bf16_to_double(gate[j])"),
    "up_dropped": ("silu(bf16_to_double(gate[j])) * bf16_to_double(up[j])", "silu(bf16_to_double(gate[j]))"),
    "row_stride_i": ("const uint16_t* gate = c + r * 2 * i;", "const uint16_t* gate = c + r * i;"),
    "up_off_by_one": ("const uint16_t* up = gate + i;", "const uint16_t* up = gate + i - 1;"),
    "decode_shift_15": ("const uint32_t u = (uint32_t)bits << 16;", "const uint32_t u = (uint32_t)bits << 15;"),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_swiglu_mistake_is_caught(name, tmp_path):
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
