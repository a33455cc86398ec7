"""Pins for the quantiser oracle's power-of-two (UE8M0) variants
(dgo_quantize_1x128_ue8m0, dgo_quantize_128x128_ue8m0 in
oracle/dg_quant_oracle.c), on the CPU, each against something other than the
oracle itself:

  * the input harness's numpy + torch quantiser with power-of-two scales (an
    independent implementation of the same rule: frexp rounding up, torch's
    e4m3 cast), read through the separately pinned unpacker;
  * closed forms: amax = 448 * 2^j gives the code 127 + j and the fp32
    quantiser's own codes; any amax a little above it the next code; an
    all-zero group code 127 and zero codes; scales 2^-130 and 1.5 * 2^-127
    (fp32 subnormals) the codes 0 and 1;
  * invariants: the scale is the smallest power of two not below amax / 448,
    every code decodes within the e4m3 rounding bound, padding bytes are 0.
Planted mistakes in copies of the oracle (rounding the exponent down, bias
128, bytes in big-endian order, the fp32 scale instead of the power of two)
must each fail one of them."""
from __future__ import annotations

import os
import subprocess

import numpy as np
import pytest

import oracle
from harness import inputs
from tests import exact_ref as X

ORACLE_DIR = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle")


def codes_of(words, groups):
    """E bytes [rows, groups] of packed words, by little-endian byte view."""
    raw = np.ascontiguousarray(words).astype("<i4").view(np.uint8).reshape(words.shape[0], -1)
    return raw[:, :groups], raw[:, groups:]


def data(rng, rows, cols):
    x = rng.standard_normal((rows, cols)).astype(np.float32)
    mag = (2.0 ** rng.integers(-20, 20, size=(rows, cols // 128))).astype(np.float32)
    return (x.reshape(rows, cols // 128, 128) * mag[:, :, None]).reshape(rows, cols)


def pin_1x128_vs_harness() -> bool:
    x = data(np.random.default_rng(21), 37, 640)
    x[3, 128:256] = 0.0
    q, w = oracle.quantize_1x128_ue8m0(x)
    qh, sh = inputs.quantize_1x128(x, pow2=True)
    return w.shape == (37, 2) and np.array_equal(q, qh) and np.array_equal(oracle.unpack_ue8m0(w, 5), sh)


def pin_128x128_vs_harness() -> bool:
    rng = np.random.default_rng(22)
    x = rng.standard_normal((300, 1152)).astype(np.float32) * np.float32(3.0)
    x[128:256, 128:256] *= np.float32(2.0 ** -30)
    x[256:, 256:384] = 0.0
    q, w = oracle.quantize_128x128_ue8m0(x)
    qh, sh = inputs.quantize_128x128(x, pow2=True)
    return w.shape == (3, 3) and np.array_equal(q, qh) and np.array_equal(oracle.unpack_ue8m0(w, 9), sh)


def pin_closed_forms() -> bool:
    rng = np.random.default_rng(23)
    j = rng.integers(-100, 100, 8)
    base = rng.uniform(-1, 1, (8, 128)).astype(np.float32)
    base[:, 7] = 1.0
    x = np.empty((8, 768), np.float32)
    for r in range(8):
        top = np.float32(448.0 * 2.0 ** j[r])
        x[r, :128] = base[r] * top                              # amax = 448 * 2^j exactly
        x[r, 128:256] = base[r] * top
        x[r, 128 + 7] = np.nextafter(top, np.float32(np.inf))  # just above: the next code
        x[r, 256:384] = 0.0                                     # all-zero group
        x[r, 384:512] = base[r] * np.float32(448.0 * 2.0 ** -130)
        x[r, 384 + 7] = np.float32(448.0 * 2.0 ** -130)         # scale 2^-130: below the E8M0 range
        x[r, 512:640] = base[r] * np.float32(448.0 * 1.5 * 2.0 ** -127)
        x[r, 512 + 7] = np.float32(448.0 * 1.5 * 2.0 ** -127)   # scale 1.5 * 2^-127: code 1
        x[r, 640:] = base[r] * np.float32(2.0 ** 100)
    q, w = oracle.quantize_1x128_ue8m0(x)
    e, pad = codes_of(w, 6)
    want = np.stack([127 + j, 128 + j, np.full(8, 127), np.zeros(8), np.ones(8)], axis=1)
    ok = np.array_equal(e[:, :5], want) and np.all(pad == 0)
    # amax = 448 * 2^j: the scale equals the fp32 quantiser's, so do the codes
    qf, sf = oracle.quantize_1x128(x[:, :128])
    ok &= np.array_equal(q[:, :128], qf) and np.array_equal(sf[:, 0], np.ldexp(np.float32(1.0), j).astype(np.float32))
    ok &= bool(np.all((q[:, 256:384] & 0x7F) == 0))
    return bool(ok)


def pin_invariants() -> bool:
    rng = np.random.default_rng(24)
    x = data(rng, 24, 512)
    q, w = oracle.quantize_1x128_ue8m0(x)
    e, _ = codes_of(w, 4)
    s = np.ldexp(1.0, e.astype(np.int64) - 127)
    amax = np.abs(x.reshape(24, 4, 128)).max(axis=2).astype(np.float64)
    s0 = (amax.astype(np.float32) / np.float32(448.0)).astype(np.float64)
    ok = bool(np.all(s >= s0)) and bool(np.all(s / 2 < s0))
    g = x.reshape(24, 4, 128).astype(np.float64)
    deq = X.torch_decode(q.reshape(24, 4, 128)).astype(np.float64) * s[:, :, None]
    bound = 2.0 ** -4 * np.abs(g) + 2.0 ** -10 * s[:, :, None] * 1.0000001
    ok &= bool(np.all(np.abs(deq - g) <= bound))
    q2, w2 = oracle.quantize_1x128_ue8m0(-x)
    ok &= np.array_equal(q2, q ^ 0x80) and np.array_equal(w2, w)
    return ok


PINS = {
    "1x128_vs_harness": pin_1x128_vs_harness,
    "128x128_vs_harness": pin_128x128_vs_harness,
    "closed_forms": pin_closed_forms,
    "invariants": pin_invariants,
}


@pytest.mark.parametrize("name", sorted(PINS))
def test_ue8m0_quantiser_pin(name):
    assert PINS[name](), name


MUTATIONS = {
    "exponent_rounded_down": ("if (ldexp(1.0, (int)e - 127) >= s0) return e;",
                              "if (ldexp(1.0, (int)e - 126) > s0) return e;"),
    "bias_128": ("double y = (double)x / ldexp(1.0, (int)e - 127);",
                 "double y = (double)x / ldexp(1.0, (int)e - 128);"),
    "big_endian_bytes": ("w |= (uint32_t)e << (8 * (g % 4));", "w |= (uint32_t)e << (8 * (3 - g % 4));"),
    "fp32_scale_kept": ("double y = (double)x / ldexp(1.0, (int)e - 127);",
                        "double y = (double)x / (double)scale_of(ldexp(448.0, (int)e - 127) * 0.75f);"),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_ue8m0_quantiser_mistake_is_caught(name, tmp_path):
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
