"""Independent exact reference used only to pin the oracle (CPU, tiny shapes).

It shares nothing with oracle/dg_oracle.c: e4m3 bytes are decoded by torch's
own float8_e4m3fn -> float64 cast (a library routine), block sums are taken in
Python/numpy integers (every e4m3 value times 2^9 is an integer), scales enter
as exact rationals (fractions.Fraction of an fp32 value is exact), and the
final rounding is a brute-force nearest search over every finite bf16 / fp32
neighbour, compared as exact rationals, ties to the even bit pattern.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np
import torch


def torch_decode(codes: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8))
    return t.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def to_int9(codes: np.ndarray) -> np.ndarray:
    v = torch_decode(codes) * 512.0
    assert np.all(np.isfinite(v)), "NaN code in operand"
    iv = v.astype(np.int64)
    assert np.array_equal(iv.astype(np.float64), v)
    return iv


def block_sums_int(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """[m, n, KB] integer block sums in units of 2^-18 (Python ints via object arrays)."""
    ai, bi = to_int9(a), to_int9(b)
    m, k = ai.shape
    n = bi.shape[0]
    kb = k // 128
    A = ai.reshape(m, kb, 128)
    B = bi.reshape(n, kb, 128)
    out = np.zeros((m, n, kb), dtype=object)
    for i in range(m):
        for j in range(n):
            for q in range(kb):
                out[i, j, q] = int(np.dot(A[i, q], B[j, q]))  # |sum| < 2^43: exact in int64
    return out


def exact_elements(a, sa, b, sb, sb_rows, kb_lo=0, kb_hi=None):
    """Exact value of sum_kb sa[i,kb]*sb[sb_rows[j],kb]*blocksum as Fractions [m][n].

    sb_rows[j] names the sb row that column j uses (j//128 for block scales,
    j for per-row scales)."""
    P = block_sums_int(a, b)
    m, n, kb = P.shape
    kb_hi = kb if kb_hi is None else kb_hi
    unit = Fraction(1, 1 << 18)
    out = [[None] * n for _ in range(m)]
    for i in range(m):
        for j in range(n):
            acc = Fraction(0)
            for q in range(kb_lo, kb_hi):
                acc += Fraction(float(sa[i, q])) * Fraction(float(sb[sb_rows[j], q])) * P[i, j, q] * unit
            out[i][j] = acc
    return out


def abs_terms(a, sa, b, sb, sb_rows):
    """sum_kb |sa*sb| * sum_k |A*B| in float64, the scale of rounding errors."""
    A = np.abs(torch_decode(a))
    B = np.abs(torch_decode(b))
    m, k = A.shape
    n = B.shape[0]
    kb = k // 128
    Ab = A.reshape(m, kb, 128)
    Bb = B.reshape(n, kb, 128)
    P = np.einsum("iqc,jqc->ijq", Ab, Bb)
    S = np.abs(sa.astype(np.float64))[:, None, :] * np.abs(sb.astype(np.float64))[np.asarray(sb_rows)][None, :, :]
    return (P * S).sum(axis=2)


# -- brute-force correct rounding -------------------------------------------

_BF16_POS = None


def _bf16_positive_table():
    global _BF16_POS
    if _BF16_POS is None:
        bits = np.arange(0, 0x7F80, dtype=np.uint32)  # +0 .. largest finite
        vals = (bits << 16).view(np.float32).astype(np.float64)
        _BF16_POS = (bits.astype(np.uint16), vals)
    return _BF16_POS


def round_bf16_exact(x: Fraction) -> int:
    """Nearest bf16 bit pattern to the exact rational x, ties to even."""
    bits, vals = _bf16_positive_table()
    neg = x < 0
    ax = -x if neg else x
    maxf = Fraction(float(vals[-1]))
    half_over = maxf + (Fraction(2) ** 128 - maxf) / 2
    if ax >= half_over:
        r = 0x7F80
    else:
        f = float(ax)
        i = int(np.searchsorted(vals, f))
        cands = [c for c in (i - 1, i, i + 1) if 0 <= c < len(vals)]
        best = None
        for c in cands:
            d = abs(Fraction(float(vals[c])) - ax)
            key = (d, int(bits[c]) & 1)
            if best is None or key < best[0]:
                best = (key, int(bits[c]))
        if ax > maxf:  # between max finite and the overflow midpoint
            best = (None, 0x7F7F)
        r = best[1]
    return r | (0x8000 if neg else 0)


def round_f32_exact(x: Fraction) -> np.float32:
    """Nearest fp32 to the exact rational x, ties to even."""
    f0 = np.float32(float(x))
    cands = {f0, np.nextafter(f0, np.float32(np.inf)), np.nextafter(f0, np.float32(-np.inf))}
    best = None
    for c in cands:
        if not np.isfinite(c):
            continue
        d = abs(Fraction(float(c)) - x)
        key = (d, int(np.array(c, np.float32).view(np.uint32)) & 1)
        if best is None or key < best[0]:
            best = (key, c)
    return np.float32(best[1])


def near_tie_bf16(x: Fraction, rel: float = 2.0 ** -40) -> bool:
    """True if x lies within rel*|x| of a bf16 rounding midpoint."""
    bits, vals = _bf16_positive_table()
    ax = abs(x)
    f = float(ax)
    i = int(np.searchsorted(vals, f))
    for c in (i - 1, i):
        if 0 <= c < len(vals) - 1:
            mid = (Fraction(float(vals[c])) + Fraction(float(vals[c + 1]))) / 2
            if abs(mid - ax) <= Fraction(rel) * ax:
                return True
    return False
