"""Pins for the BF16 NT GEMM oracle (dgo_gemm_bf16_nt in oracle/dg_oracle.c), on
the CPU, each against something other than the oracle itself: torch's bf16
decode (a library routine), an exact rational brute force with a correctly
rounded bf16 result (tests/exact_ref.py), numpy's fp64 matmul, and closed
forms.  Planted mistakes in copies of the oracle must each fail a pin."""
from __future__ import annotations

import os
import subprocess
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from tests import exact_ref as X

ORACLE_DIR = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle")


def torch_bf16_value(bits: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(bits, np.uint16).view(np.int16)).view(torch.bfloat16) \
        .to(torch.float64).numpy()


def rand_bf16(rng, shape, lo=-8, hi=8):
    """Finite bf16 bit patterns of N(0,1) values times 2^U(lo, hi)."""
    x = (rng.standard_normal(shape) * 2.0 ** rng.integers(lo, hi, shape)).astype(np.float32)
    return torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def pin_decode_identity() -> bool:
    """K = 1 with B = 1.0: C is A itself (an exact bf16 value rounds to itself)."""
    rng = np.random.default_rng(1)
    a = rng.integers(0, 1 << 16, size=(4096, 1), dtype=np.uint16)
    a = a[(a & 0x7F80) != 0x7F80].reshape(-1, 1)  # finite patterns only
    c, x = oracle.gemm_bf16_nt(a, np.array([[0x3F80]], np.uint16))
    ok = np.array_equal(x[:, 0], torch_bf16_value(a[:, 0]))
    # -0 and +0 both give +0 after the fp64 sum 0.0 + (-0 * 1) = +0
    nz = torch_bf16_value(a[:, 0]) != 0
    return ok and np.array_equal(c[nz, 0], a[nz, 0])


def pin_brute_force() -> bool:
    rng = np.random.default_rng(2)
    ok = True
    for (m, n, k) in [(3, 5, 7), (2, 17, 64), (4, 3, 130)]:
        a, b = rand_bf16(rng, (m, k)), rand_bf16(rng, (n, k))
        c, _ = oracle.gemm_bf16_nt(a, b)
        av, bv = torch_bf16_value(a), torch_bf16_value(b)
        for i in range(m):
            for j in range(n):
                ex = sum((Fraction(float(av[i, t])) * Fraction(float(bv[j, t])) for t in range(k)), Fraction(0))
                if not X.near_tie_bf16(ex) and int(c[i, j]) != X.round_bf16_exact(ex):
                    ok = False
    return ok


def pin_numpy_matmul() -> bool:
    rng = np.random.default_rng(3)
    a, b = rand_bf16(rng, (40, 384)), rand_bf16(rng, (50, 384))
    _, x = oracle.gemm_bf16_nt(a, b)
    av, bv = torch_bf16_value(a), torch_bf16_value(b)
    ref = av @ bv.T
    scale = np.abs(av) @ np.abs(bv).T
    return bool(np.all(np.abs(x - ref) <= 1e-12 * scale + 1e-300))


def pin_closed_forms() -> bool:
    k = 7168
    ones = np.full((3, k), 0x3F80, np.uint16)
    c, _ = oracle.gemm_bf16_nt(ones, ones[:2])
    ok = bool(np.all(c == 0x45E0))  # 7168.0
    rng = np.random.default_rng(4)
    # small integers: every sum is exact, so negation and K permutation act exactly
    a = torch.from_numpy(rng.integers(-8, 9, (5, 256)).astype(np.float32)).to(torch.bfloat16) \
        .view(torch.int16).numpy().view(np.uint16)
    b = torch.from_numpy(rng.integers(-8, 9, (6, 256)).astype(np.float32)).to(torch.bfloat16) \
        .view(torch.int16).numpy().view(np.uint16)
    c0, x0 = oracle.gemm_bf16_nt(a, b)
    _, x1 = oracle.gemm_bf16_nt(a ^ np.uint16(0x8000), b)
    perm = rng.permutation(256)
    _, x2 = oracle.gemm_bf16_nt(a[:, perm], b[:, perm])
    ok &= np.array_equal(x1, -x0) and np.array_equal(x2, x0)
    ok &= np.array_equal(x0, torch_bf16_value(a) @ torch_bf16_value(b).T)
    return ok


def pin_sampled_matches_full() -> bool:
    rng = np.random.default_rng(5)
    a, b = rand_bf16(rng, (33, 256)), rand_bf16(rng, (40, 256))
    _, x = oracle.gemm_bf16_nt(a, b)
    r, c = rng.integers(0, 33, 200), rng.integers(0, 40, 200)
    return np.array_equal(oracle.gemm_bf16_nt_at(a, b, r, c), x[r, c])


PINS = {"decode_identity": pin_decode_identity, "brute_force": pin_brute_force,
        "numpy_matmul": pin_numpy_matmul, "closed_forms": pin_closed_forms,
        "sampled_matches_full": pin_sampled_matches_full}


@pytest.mark.parametrize("name", sorted(PINS))
def test_bf16_oracle_pin(name):
    assert PINS[name](), name


MUTATIONS = {
    "dropped_last_product": ("for (int64_t t = 0; t < k; ++t) acc += bf16_value",
                             "for (int64_t t = 0; t < k - 1; ++t) acc += bf16_value"),
    "decode_shift_15": ("const uint32_t u = (uint32_t)h << 16;", "const uint32_t u = (uint32_t)h << 15;"),
    "b_row_of_a": ("bf16_element(a + i * k, b + j * k, k)", "bf16_element(a + i * k, b + i * k, k)"),
    "sampled_swapped": ("bf16_element(a + rows[i] * k, b + cols[i] * k, k)",
                        "bf16_element(a + cols[i] * k, b + rows[i] * k, k)"),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_bf16_mistake_is_caught(name, tmp_path):
    old, new = MUTATIONS[name]
    src = open(os.path.join(ORACLE_DIR, "dg_oracle.c")).read()
    assert src.count(old) == 1, f"mutation anchor for {name} not found"
    (tmp_path / "o.c").write_text(src.replace(old, new))
    so = tmp_path / "libmut.so"
    subprocess.run(["gcc", "-O1", "-ffp-contract=off", "-fopenmp", "-shared", "-fPIC", "-o", str(so),
                    str(tmp_path / "o.c"), os.path.join(ORACLE_DIR, "dg_quant_oracle.c"), "-lm"], check=True)
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


# ---- the grouped BF16 compositions (oracle.grouped_contiguous_bf16 / _masked_bf16) ----

def test_grouped_bf16_compositions_against_the_dense_oracle():
    """One expert owning every row is the dense oracle; padding rows, ids past
    G and rows past masked_m keep their initial bits; renumbering the experts
    (ids and B slices alike) leaves the result unchanged; masked_m beyond M_max
    is M_max."""
    from harness import inputs
    x = inputs.make_contiguous_bf16(3, 128, 70, 192, seed=inputs.SEED_BASE + 40, max_pad=60)
    init = np.full((x.a.shape[0], 70), 0xFFFF, np.uint16)
    ones = np.zeros(x.a.shape[0], np.int32)
    c1, _ = oracle.grouped_contiguous_bf16(x.a, x.b[:1], ones, init)
    d1, _ = oracle.gemm_bf16_nt(x.a, x.b[0])
    assert np.array_equal(c1, d1)
    ids = x.ctrl.copy()
    ids[:7] = 9                                     # past G: skipped
    c, _ = oracle.grouped_contiguous_bf16(x.a, x.b, ids, init)
    keep = (ids < 0) | (ids >= 3)
    assert np.all(c[keep] == 0xFFFF) and not np.any(c[~keep] == 0xFFFF)
    perm = np.array([2, 0, 1])                     # expert e becomes perm[e]
    ids2 = np.where((ids >= 0) & (ids < 3), perm[np.clip(ids, 0, 2)], ids).astype(np.int32)
    b2 = np.empty_like(x.b)
    b2[perm] = x.b
    c2, _ = oracle.grouped_contiguous_bf16(x.a, b2, ids2, init)
    assert np.array_equal(c, c2)
    y = inputs.make_masked_bf16(3, 40, 50, 128, seed=inputs.SEED_BASE + 41, masked_m=[0, 17, 99])
    init = np.full((3, 40, 50), 0xFFFF, np.uint16)
    cm, _ = oracle.grouped_masked_bf16(y.a, y.b, y.ctrl, init)
    assert np.all(cm[0] == 0xFFFF) and np.all(cm[1, 17:] == 0xFFFF)
    assert np.array_equal(cm[1, :17], oracle.gemm_bf16_nt(y.a[1, :17], y.b[1])[0])
    assert np.array_equal(cm[2], oracle.gemm_bf16_nt(y.a[2], y.b[2])[0])
