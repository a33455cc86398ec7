"""Python front of the CPU oracle (dg_oracle.c).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's
CPU-baseline leg may import this package; the library and its Python binding
never do.  It shares no code with the HIP path.  All arrays are host numpy
arrays; fp8 operands are uint8 e4m3fn bytes, bf16 results are uint16 bit
patterns, and every "exact" result is the fp64 value before the single final
rounding (see dg_oracle.c for the definition and the pages it follows).
"""
from __future__ import annotations

import contextlib
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "dg_oracle.c")
_SRCS = [_SRC, os.path.join(_HERE, "dg_quant_oracle.c")]
_LIB = os.path.join(_HERE, "libdg_oracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile dg_oracle.c into oracle/libdg_oracle.so with gcc + OpenMP."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        cmd = ["gcc", "-O2", "-ffp-contract=off", "-fopenmp", "-shared", "-fPIC",
               "-o", tmp, *_SRCS, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        _lib = ctypes.CDLL(_LIB)
    return _lib


@contextlib.contextmanager
def using_library(path: str):
    """Temporarily route every call to another build of dg_oracle.c (used by
    the tests that plant mistakes in a copy of the oracle)."""
    global _lib
    old = _lib
    _lib = ctypes.CDLL(path)
    try:
        yield
    finally:
        _lib = old


_P = ctypes.c_void_p
_I = ctypes.c_int64


def _p(x):
    return None if x is None else ctypes.c_void_p(x.ctypes.data)


def _c(x, dtype):
    return np.ascontiguousarray(x, dtype=dtype)


def _check(rc, what):
    if rc < 0:
        raise ValueError(f"oracle {what}: invalid arguments (rc={rc})")
    return rc


def num_threads() -> int:
    """Threads the OpenMP runtime will use (OMP_NUM_THREADS or all cores)."""
    v = os.environ.get("OMP_NUM_THREADS")
    return int(v) if v else (os.cpu_count() or 1)


def e4m3_table() -> np.ndarray:
    out = np.empty(256, np.float64)
    lib().dgo_e4m3_table(_p(out))
    return out


def round_bf16(x: np.ndarray) -> np.ndarray:
    x = _c(x, np.float64)
    out = np.empty(x.shape, np.uint16)
    lib().dgo_round_bf16(_p(x), _p(out), _I(x.size))
    return out


def round_f32(x: np.ndarray) -> np.ndarray:
    x = _c(x, np.float64)
    out = np.empty(x.shape, np.float32)
    lib().dgo_round_f32(_p(x), _p(out), _I(x.size))
    return out


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float32 values (exact widening)."""
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32)


def block_sums_f64(a, b):
    a, b = _c(a, np.uint8), _c(b, np.uint8)
    m, k = a.shape
    n = b.shape[0]
    out = np.empty((m, n, k // 128), np.float64)
    _check(lib().dgo_block_sums_f64(_p(a), _p(b), _I(m), _I(n), _I(k), _p(out)), "block_sums_f64")
    return out


def block_sums_i64(a, b):
    """(sums in units of 2^-18, nan_seen)."""
    a, b = _c(a, np.uint8), _c(b, np.uint8)
    m, k = a.shape
    n = b.shape[0]
    out = np.empty((m, n, k // 128), np.int64)
    rc = _check(lib().dgo_block_sums_i64(_p(a), _p(b), _I(m), _I(n), _I(k), _p(out)),
                "block_sums_i64")
    return out, bool(rc)


def gemm_fp8_nt(a, sa, b, sb):
    """Dense: returns (C bf16 bits [M,N], exact fp64 [M,N])."""
    a, b = _c(a, np.uint8), _c(b, np.uint8)
    sa, sb = _c(sa, np.float32), _c(sb, np.float32)
    m, k = a.shape
    n = b.shape[0]
    c = np.empty((m, n), np.uint16)
    x = np.empty((m, n), np.float64)
    _check(lib().dgo_gemm_fp8_nt(_p(a), _p(sa), _p(b), _p(sb), _I(m), _I(n), _I(k), _p(c), _p(x)),
           "gemm_fp8_nt")
    return c, x


def gemm_fp8_nt_at(a, sa, b, sb, rows, cols):
    a, b = _c(a, np.uint8), _c(b, np.uint8)
    sa, sb = _c(sa, np.float32), _c(sb, np.float32)
    rows, cols = _c(rows, np.int64), _c(cols, np.int64)
    m, k = a.shape
    n = b.shape[0]
    out = np.empty(rows.shape, np.float64)
    _check(lib().dgo_gemm_fp8_nt_at(_p(a), _p(sa), _p(b), _p(sb), _I(m), _I(n), _I(k),
                                    _p(rows), _p(cols), _I(rows.size), _p(out)), "gemm_fp8_nt_at")
    return out


def unpack_ue8m0(words, kblocks: int) -> np.ndarray:
    """Packed UE8M0 scales -> fp32 scale values [R, kblocks].

    DeepGEMM pages (aikraft.ru, support table): the scale format of the newer
    architecture is packed UE8M0, four values in one torch.int.  Read here as:
    word w of a row holds the scales of K blocks 4w..4w+3, K block 4w+i in
    byte i (little-endian, bits 8i..8i+7); a byte E is the unsigned 8-bit
    exponent of the E8M0 format, scale 2^(E - 127), with E = 255 the format's
    NaN.  Bytes past `kblocks` are padding and ignored.  Every 2^(E - 127) for
    E <= 254 is an fp32 value (2^-127 a subnormal), so the result is exact.
    """
    words = np.asarray(words)
    lead = words.shape[:-1]
    w = np.ascontiguousarray(words).reshape(-1, words.shape[-1]).astype(np.int64) & 0xFFFFFFFF
    r, kw = w.shape
    assert 4 * kw >= kblocks, "too few words for the K blocks"
    out = np.empty((r, kblocks), np.float64)
    for kb in range(kblocks):
        e = (w[:, kb // 4] >> (8 * (kb % 4))) & 0xFF
        out[:, kb] = np.where(e == 255, np.nan, np.ldexp(1.0, (e - 127).astype(np.int32)))
    return out.astype(np.float32).reshape(*lead, kblocks)


def gemm_fp8_nt_ue8m0_packed(a, sa_words, b, sb_words):
    """Dense GEMM with packed UE8M0 scales: the scales unpacked, then the
    dense oracle (the packed format only encodes power-of-two fp32 scales)."""
    kb = np.asarray(a).shape[1] // 128
    return gemm_fp8_nt(a, unpack_ue8m0(sa_words, kb), b, unpack_ue8m0(sb_words, kb))


def grouped_contiguous_ue8m0_packed(a, sa_words, b, sb_words, m_indices, c_init):
    """Contiguous MoE with packed UE8M0 scales: unpacked, then grouped_contiguous."""
    kb = np.asarray(a).shape[1] // 128
    return grouped_contiguous(a, unpack_ue8m0(sa_words, kb), b, unpack_ue8m0(sb_words, kb), m_indices, c_init)


def grouped_masked_ue8m0_packed(a, sa_words, b, sb_words, masked_m, c_init):
    """Masked MoE with packed UE8M0 scales: unpacked, then grouped_masked."""
    kb = np.asarray(a).shape[2] // 128
    return grouped_masked(a, unpack_ue8m0(sa_words, kb), b, unpack_ue8m0(sb_words, kb), masked_m, c_init)


def grouped_contiguous(a, sa, b, sb, m_indices, c_init):
    """Contiguous MoE: returns (C bits with valid rows written over c_init, exact fp64)."""
    a, b = _c(a, np.uint8), _c(b, np.uint8)
    sa, sb = _c(sa, np.float32), _c(sb, np.float32)
    ids = _c(m_indices, np.int32)
    m_total, k = a.shape
    g, n, _ = b.shape
    c = np.array(c_init, dtype=np.uint16, copy=True, order="C")
    x = np.full((m_total, n), np.nan, np.float64)
    _check(lib().dgo_grouped_contiguous(_p(a), _p(sa), _p(b), _p(sb), _p(ids), _I(m_total),
                                        _I(n), _I(k), _I(g), _p(c), _p(x)), "grouped_contiguous")
    return c, x


def grouped_contiguous_at(a, sa, b, sb, m_indices, rows, cols):
    a, b = _c(a, np.uint8), _c(b, np.uint8)
    sa, sb = _c(sa, np.float32), _c(sb, np.float32)
    ids = _c(m_indices, np.int32)
    rows, cols = _c(rows, np.int64), _c(cols, np.int64)
    m_total, k = a.shape
    g, n, _ = b.shape
    out = np.empty(rows.shape, np.float64)
    wr = np.empty(rows.shape, np.int8)
    _check(lib().dgo_grouped_contiguous_at(_p(a), _p(sa), _p(b), _p(sb), _p(ids), _I(m_total),
                                           _I(n), _I(k), _I(g), _p(rows), _p(cols),
                                           _I(rows.size), _p(out), _p(wr)),
           "grouped_contiguous_at")
    return out, wr.astype(bool)


def grouped_masked(a, sa, b, sb, masked_m, c_init):
    """Masked MoE: a [G,M_max,K]; returns (C bits [G,M_max,N] over c_init, exact fp64)."""
    a, b = _c(a, np.uint8), _c(b, np.uint8)
    sa, sb = _c(sa, np.float32), _c(sb, np.float32)
    mm = _c(masked_m, np.int32)
    g, m_max, k = a.shape
    n = b.shape[1]
    c = np.array(c_init, dtype=np.uint16, copy=True, order="C")
    x = np.full((g, m_max, n), np.nan, np.float64)
    _check(lib().dgo_grouped_masked(_p(a), _p(sa), _p(b), _p(sb), _p(mm), _I(g), _I(m_max),
                                    _I(n), _I(k), _p(c), _p(x)), "grouped_masked")
    return c, x


def grouped_masked_at(a, sa, b, sb, masked_m, groups, rows, cols):
    a, b = _c(a, np.uint8), _c(b, np.uint8)
    sa, sb = _c(sa, np.float32), _c(sb, np.float32)
    mm = _c(masked_m, np.int32)
    groups, rows, cols = _c(groups, np.int64), _c(rows, np.int64), _c(cols, np.int64)
    g, m_max, k = a.shape
    n = b.shape[1]
    out = np.empty(rows.shape, np.float64)
    wr = np.empty(rows.shape, np.int8)
    _check(lib().dgo_grouped_masked_at(_p(a), _p(sa), _p(b), _p(sb), _p(mm), _I(g), _I(m_max),
                                       _I(n), _I(k), _p(groups), _p(rows), _p(cols),
                                       _I(rows.size), _p(out), _p(wr)), "grouped_masked_at")
    return out, wr.astype(bool)


def wgrad(a, sa, b, sb, d0):
    """Weight gradient: returns (D fp32 = fp32(D0 + sum), exact fp64)."""
    a, b = _c(a, np.uint8), _c(b, np.uint8)
    sa, sb = _c(sa, np.float32), _c(sb, np.float32)
    m, k = a.shape
    n = b.shape[0]
    d = np.array(d0, dtype=np.float32, copy=True, order="C").reshape(m, n)
    x = np.empty((m, n), np.float64)
    _check(lib().dgo_wgrad(_p(a), _p(sa), _p(b), _p(sb), _I(m), _I(n), _I(k), _p(d), _p(x)),
           "wgrad")
    return d, x


def wgrad_at(a, sa, b, sb, d0, rows, cols):
    a, b = _c(a, np.uint8), _c(b, np.uint8)
    sa, sb = _c(sa, np.float32), _c(sb, np.float32)
    rows, cols = _c(rows, np.int64), _c(cols, np.int64)
    m, k = a.shape
    n = b.shape[0]
    d0c = None if d0 is None else _c(d0, np.float32)
    out = np.empty(rows.shape, np.float64)
    _check(lib().dgo_wgrad_at(_p(a), _p(sa), _p(b), _p(sb), _I(m), _I(n), _I(k), _p(d0c),
                              _p(rows), _p(cols), _I(rows.size), _p(out)), "wgrad_at")
    return out


def k_grouped_wgrad(a, sa, b, sb, ks, d0):
    """K-grouped weight gradient: D fp32 [G,M,N]; returns (D_new, exact fp64)."""
    a, b = _c(a, np.uint8), _c(b, np.uint8)
    sa, sb = _c(sa, np.float32), _c(sb, np.float32)
    ks = _c(ks, np.int64)
    m = a.shape[0]
    n = b.shape[0]
    g = ks.size
    d = np.array(d0, dtype=np.float32, copy=True, order="C").reshape(g, m, n)
    x = np.empty((g, m, n), np.float64)
    _check(lib().dgo_k_grouped_wgrad(_p(a), _p(sa), _p(b), _p(sb), _p(ks), _I(g), _I(m), _I(n),
                                     _p(d), _p(x)), "k_grouped_wgrad")
    return d, x


def k_grouped_wgrad_at(a, sa, b, sb, ks, d0, groups, rows, cols):
    a, b = _c(a, np.uint8), _c(b, np.uint8)
    sa, sb = _c(sa, np.float32), _c(sb, np.float32)
    ks = _c(ks, np.int64)
    groups, rows, cols = _c(groups, np.int64), _c(rows, np.int64), _c(cols, np.int64)
    m = a.shape[0]
    n = b.shape[0]
    d0c = None if d0 is None else _c(d0, np.float32)
    out = np.empty(rows.shape, np.float64)
    _check(lib().dgo_k_grouped_wgrad_at(_p(a), _p(sa), _p(b), _p(sb), _p(ks), _I(ks.size), _I(m),
                                        _I(n), _p(d0c), _p(groups), _p(rows), _p(cols),
                                        _I(rows.size), _p(out)), "k_grouped_wgrad_at")
    return out


# ---- FP8 quantiser (dg_quant_oracle.c) ----

def e4m3_encode(y: np.ndarray) -> np.ndarray:
    """fp32 values (|y| <= 448) -> nearest e4m3fn codes, ties to even."""
    y = _c(y, np.float32)
    out = np.empty(y.shape, np.uint8)
    lib().dgo_e4m3_encode(_p(y), _p(out), _I(y.size))
    return out


def quantize_1x128(x: np.ndarray):
    """x fp32 [M,K] -> (q uint8 [M,K], s fp32 [M,K/128])."""
    x = _c(x, np.float32)
    m, k = x.shape
    q = np.empty((m, k), np.uint8)
    s = np.empty((m, k // 128), np.float32)
    _check(lib().dgo_quantize_1x128(_p(x), _I(m), _I(k), _p(q), _p(s)), "quantize_1x128")
    return q, s


def quantize_128x128(x: np.ndarray):
    """x fp32 [N,K] -> (q uint8 [N,K], s fp32 [ceil(N/128),K/128])."""
    x = _c(x, np.float32)
    n, k = x.shape
    q = np.empty((n, k), np.uint8)
    s = np.empty(((n + 127) // 128, k // 128), np.float32)
    _check(lib().dgo_quantize_128x128(_p(x), _I(n), _I(k), _p(q), _p(s)), "quantize_128x128")
    return q, s


def quantize_1x128_ue8m0(x: np.ndarray):
    """x fp32 [M,K] -> (q uint8 [M,K], packed UE8M0 codes int32 [M,ceil(K/512)]):
    the smallest power-of-two scale not below amax/448 per 1x128 group."""
    x = _c(x, np.float32)
    m, k = x.shape
    q = np.empty((m, k), np.uint8)
    s = np.empty((m, (k // 128 + 3) // 4), np.int32)
    _check(lib().dgo_quantize_1x128_ue8m0(_p(x), _I(m), _I(k), _p(q), _p(s)), "quantize_1x128_ue8m0")
    return q, s


def quantize_128x128_ue8m0(x: np.ndarray):
    """x fp32 [N,K] -> (q uint8 [N,K], packed UE8M0 codes int32 [ceil(N/128),ceil(K/512)])."""
    x = _c(x, np.float32)
    n, k = x.shape
    q = np.empty((n, k), np.uint8)
    s = np.empty(((n + 127) // 128, (k // 128 + 3) // 4), np.int32)
    _check(lib().dgo_quantize_128x128_ue8m0(_p(x), _I(n), _I(k), _p(q), _p(s)), "quantize_128x128_ue8m0")
    return q, s


def quantize_1x128_transposed(x: np.ndarray):
    """x fp32 [T,F] -> (q uint8 [F,T], s fp32 [F,T/128]): 1x128 groups along T."""
    x = _c(x, np.float32)
    t, f = x.shape
    q = np.empty((f, t), np.uint8)
    s = np.empty((f, t // 128), np.float32)
    _check(lib().dgo_quantize_1x128_transposed(_p(x), _I(t), _I(f), _p(q), _p(s)),
           "quantize_1x128_transposed")
    return q, s


# ---- BF16 NT GEMM (dg_oracle.c) ----

def gemm_bf16_nt(a, b):
    """A [M,K], B [N,K] bf16 bit patterns (uint16) -> (C bf16 bits [M,N], exact-sum fp64 [M,N])."""
    a, b = _c(a, np.uint16), _c(b, np.uint16)
    m, k = a.shape
    n = b.shape[0]
    c = np.empty((m, n), np.uint16)
    x = np.empty((m, n), np.float64)
    _check(lib().dgo_gemm_bf16_nt(_p(a), _p(b), _I(m), _I(n), _I(k), _p(c), _p(x)), "gemm_bf16_nt")
    return c, x


def gemm_bf16_nt_at(a, b, rows, cols):
    """Unrounded fp64 values of the sampled outputs (rows[i], cols[i])."""
    a, b = _c(a, np.uint16), _c(b, np.uint16)
    rows, cols = _c(rows, np.int64), _c(cols, np.int64)
    m, k = a.shape
    n = b.shape[0]
    out = np.empty(rows.shape, np.float64)
    _check(lib().dgo_gemm_bf16_nt_at(_p(a), _p(b), _I(m), _I(n), _I(k), _p(rows), _p(cols), _I(rows.size),
                                     _p(out)), "gemm_bf16_nt_at")
    return out


def grouped_contiguous_bf16(a, b, m_indices, c_init):
    """Contiguous MoE in BF16: the rows whose expert id is e in [0, G) are the
    BF16 oracle's product of those rows of A with B[e]; every other row keeps
    c_init.  Returns (C bf16 bits, exact fp64 with NaN on untouched rows)."""
    a, b = np.asarray(a, np.uint16), np.asarray(b, np.uint16)
    ids = np.asarray(m_indices)
    c = np.array(c_init, np.uint16, copy=True)
    x = np.full(c.shape, np.nan)
    for e in range(b.shape[0]):
        rows = np.flatnonzero(ids == e)
        if rows.size:
            c[rows], x[rows] = gemm_bf16_nt(a[rows], b[e])
    return c, x


def grouped_masked_bf16(a, b, masked_m, c_init):
    """Masked MoE in BF16: rows r < clamp(masked_m[g], 0, M_max) of group g are
    the BF16 oracle's product of A[g, :r] with B[g]; other rows keep c_init."""
    a, b = np.asarray(a, np.uint16), np.asarray(b, np.uint16)
    c = np.array(c_init, np.uint16, copy=True)
    x = np.full(c.shape, np.nan)
    for g in range(a.shape[0]):
        v = int(min(max(int(masked_m[g]), 0), a.shape[1]))
        if v:
            c[g, :v], x[g, :v] = gemm_bf16_nt(a[g, :v], b[g])
    return c, x


# ---- SwiGLU then 1x128 quantise (dg_quant_oracle.c) ----

def swiglu_quantize_1x128(c: np.ndarray):
    """c bf16 bits (uint16) [M, 2I], gate = c[:, :I], up = c[:, I:] ->
    (q uint8 [M, I], s fp32 [M, I/128], h fp64 [M, I] before its fp32 rounding)."""
    c = _c(c, np.uint16)
    m, i2 = c.shape
    i = i2 // 2
    q = np.empty((m, i), np.uint8)
    s = np.empty((m, i // 128), np.float32)
    h = np.empty((m, i), np.float64)
    _check(lib().dgo_swiglu_quantize_1x128(_p(c), _I(m), _I(i), _p(q), _p(s), _p(h)), "swiglu_quantize_1x128")
    return q, s, h
