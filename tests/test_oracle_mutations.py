"""Plant plausible mistakes in copies of the oracle (on the CPU) and check that
the pins catch every one: a dropped term, a wrong sign, a wrong exponent bias,
a wrong scale index, a transposed scale, truncation instead of
round-to-nearest-even, the wrong expert, an off-by-one masked row, a lost D0
and a K-group offset that is never advanced.  The real oracle passes the same
pins (test_oracle.py), so each failure below is the mutation's doing.
"""
from __future__ import annotations

import os
import subprocess
from fractions import Fraction

import numpy as np
import pytest

import oracle
from tests import exact_ref as X

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "dg_oracle.c")

MUTATIONS = {
    "dropped_last_product": ("for (int64_t k = kb * BK; k < (kb + 1) * BK; ++k)",
                             "for (int64_t k = kb * BK; k < (kb + 1) * BK - 1; ++k)"),
    "sign_ignored": ("return s ? -mag : mag;", "return mag;"),
    "exponent_bias_8": ("(int)e - 7);", "(int)e - 8);"),
    "subnormal_exponent": ("ldexp((double)f / 8.0, -6)", "ldexp((double)f / 8.0, -7)"),
    "sb_block_ignored_dense": ("sb + (j / BK) * KB, 0, KB);\n      if (c_exact) c_exact[i * n + j]",
                               "sb + 0 * KB, 0, KB);\n      if (c_exact) c_exact[i * n + j]"),
    "scale_first_block_only": ("double s = (double)sa_row[kb] * (double)sb_row[kb];",
                               "double s = (double)sa_row[kb] * (double)sb_row[kb0];"),
    "truncating_round": ("y = nearbyint(ldexp(ax, 7 - e));", "y = floor(ldexp(ax, 7 - e));"),
    "contiguous_expert_zero": ("double v = element(a + r * k, sa + r * KB, b + (e * n + j) * k,",
                               "double v = element(a + r * k, sa + r * KB, b + (0 * n + j) * k,"),
    "masked_off_by_one": ("if (r >= valid_rows(masked_m, gi, m_max)) continue;",
                          "if (r > valid_rows(masked_m, gi, m_max)) continue;"),
    "wgrad_d0_dropped": ("double v = (double)d[i * n + j] +", "double v = 0.0 +"),
    "kgroup_offset_stuck": ("    kb0 = kb1;\n", "    kb0 = kb0;\n"),
}


def _rng_codes(rng, shape):
    c = rng.integers(0, 256, size=shape, dtype=np.uint8)
    c[(c & 0x7F) == 0x7F] = 0x7E
    return c


def _scales(rng, shape):
    return (2.0 ** rng.uniform(-6, 6, size=shape)).astype(np.float32)


def _bits_ok(c, ex):
    for idx, e in np.ndenumerate(np.asarray(ex, dtype=object)):
        if not X.near_tie_bf16(e) and int(c[idx]) != X.round_bf16_exact(e):
            return False
    return True


def run_pins() -> list:
    """Compact exact-value pins over every kind; returns the names that fail."""
    failed = []
    rng = np.random.default_rng(777)
    # decode table vs torch
    t = oracle.e4m3_table()
    ref = X.torch_decode(np.arange(256, dtype=np.uint8))
    fin = np.isfinite(ref)
    if not (np.array_equal(np.isnan(t), ~fin) and np.array_equal(t[fin], ref[fin])):
        failed.append("decode")
    # rounding vs torch on fp32 inputs
    x = (rng.standard_normal(2000) * 2.0 ** rng.integers(-20, 20, 2000)).astype(np.float32)
    import torch
    if not np.array_equal(oracle.round_bf16(x.astype(np.float64)),
                          torch.from_numpy(x).to(torch.bfloat16).view(torch.uint16).numpy()):
        failed.append("round")
    # dense, N tail across two scale blocks
    m, n, k = 3, 130, 256
    a, b = _rng_codes(rng, (m, k)), _rng_codes(rng, (n, k))
    sa, sb = _scales(rng, (m, 2)), _scales(rng, (2, 2))
    c, _ = oracle.gemm_fp8_nt(a, sa, b, sb)
    if not _bits_ok(c, X.exact_elements(a, sa, b, sb, [j // 128 for j in range(n)])):
        failed.append("dense")
    # contiguous
    g = 2
    ids = np.array([1, 0, -1, 1], np.int32)
    a, bg = _rng_codes(rng, (4, k)), _rng_codes(rng, (g, 5, k))
    sa, sbg = _scales(rng, (4, 2)), _scales(rng, (g, 1, 2))
    c, _ = oracle.grouped_contiguous(a, sa, bg, sbg, ids, np.full((4, 5), 0xFFFF, np.uint16))
    ok = np.all(c[2] == 0xFFFF)
    for r in (0, 1, 3):
        e = ids[r]
        ok &= _bits_ok(c[r:r + 1], X.exact_elements(a[r:r + 1], sa[r:r + 1], bg[e], sbg[e], [0] * 5))
    if not ok:
        failed.append("contiguous")
    # masked
    mm = np.array([2, 0], np.int32)
    a3, bg = _rng_codes(rng, (g, 3, k)), _rng_codes(rng, (g, 4, k))
    sa3, sbg = _scales(rng, (g, 3, 2)), _scales(rng, (g, 1, 2))
    c, _ = oracle.grouped_masked(a3, sa3, bg, sbg, mm, np.full((g, 3, 4), 0xFFFF, np.uint16))
    ok = np.all(c[0, 2:] == 0xFFFF) and np.all(c[1] == 0xFFFF)
    ok &= _bits_ok(c[0, :2], X.exact_elements(a3[0, :2], sa3[0, :2], bg[0], sbg[0], [0] * 4))
    if not ok:
        failed.append("masked")
    # wgrad with D0
    a, b = _rng_codes(rng, (2, k)), _rng_codes(rng, (3, k))
    sa, sb = _scales(rng, (2, 2)), _scales(rng, (3, 2))
    d0 = rng.standard_normal((2, 3)).astype(np.float32)
    d, _ = oracle.wgrad(a, sa, b, sb, d0)
    ex = X.exact_elements(a, sa, b, sb, [0, 1, 2])
    if not all(d[i, j] == X.round_f32_exact(Fraction(float(d0[i, j])) + ex[i][j])
               for i in range(2) for j in range(3)):
        failed.append("wgrad")
    # k-grouped wgrad
    ks = [128, 128]
    d0 = rng.standard_normal((2, 2, 3)).astype(np.float32)
    d, _ = oracle.k_grouped_wgrad(a, sa, b, sb, ks, d0)
    ok = True
    for gi in range(2):
        ex = X.exact_elements(a, sa, b, sb, [0, 1, 2], gi, gi + 1)
        ok &= all(d[gi, i, j] == X.round_f32_exact(Fraction(float(d0[gi, i, j])) + ex[i][j])
                  for i in range(2) for j in range(3))
    if not ok:
        failed.append("k_grouped")
    return failed


def test_real_oracle_passes_compact_pins():
    assert run_pins() == []


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name, tmp_path):
    old, new = MUTATIONS[name]
    src = open(SRC).read()
    assert src.count(old) >= 1, f"mutation anchor for {name} not found"
    mutated = src.replace(old, new)
    cpath = tmp_path / "mut.c"
    cpath.write_text(mutated)
    so = tmp_path / "libmut.so"
    subprocess.run(["gcc", "-O1", "-ffp-contract=off", "-fopenmp", "-shared", "-fPIC", "-o", str(so),
                    str(cpath), "-lm"], check=True)
    with oracle.using_library(str(so)):
        failed = run_pins()
    assert failed, f"planted mistake {name} was not caught by any pin"
