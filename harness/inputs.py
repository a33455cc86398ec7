"""Seeded synthetic inputs shared by the HIP path's tests/bench and by the oracle.

This module only *makes inputs*: random fp32 data, its quantisation to FP8 e4m3
bytes plus fp32 scale factors, expert ids and masked row counts.  It holds none
of the GEMM's arithmetic (no decode, no products, no accumulation, no output
rounding), so the oracle and the GPU path can both consume its bytes without
sharing any of the method's code.

Quantisation follows the fine-grained scaling the DeepGEMM pages describe
(DeepSeek DeepGEMM 中文讲解, "使用示例": activations carry one fp32 scale per
row and 128-wide K block, shape [M, K/128]; weights one per 128x128 block,
shape [ceil(N/128), K/128]; "注意事项": FP8 needs dynamic scale factors from
amax).  Per group: amax = max |x|, s = amax / 448 (448 = largest finite e4m3
value), q = e4m3(clamp(x / s, +-448)) with round-to-nearest-even; an all-zero
group gets s = 1.  The e4m3 encoding is torch's CPU cast to float8_e4m3fn
(OCP E4M3FN), a library routine; the clamp is needed because that cast does not
saturate (470 becomes NaN).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch

SEED_BASE = 20250226
E4M3_MAX = 448.0
BLOCK_K = 128


def _rng(seed: int, stream: int) -> np.random.Generator:
    """Child stream `stream` of SeedSequence(seed) (PCG64)."""
    ss = np.random.SeedSequence(seed)
    return np.random.Generator(np.random.PCG64(ss.spawn(stream + 1)[stream]))


def _encode_e4m3(y: np.ndarray) -> np.ndarray:
    """fp32 values already in [-448, 448] -> e4m3fn bytes (RNE), via torch's CPU cast."""
    t = torch.from_numpy(np.ascontiguousarray(y, dtype=np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def _pow2_ceil(s: np.ndarray) -> np.ndarray:
    """The smallest power of two >= s (s > 0, fp32): UE8M0-representable scales."""
    m, e = np.frexp(s.astype(np.float64))
    return np.ldexp(1.0, np.where(m == 0.5, e - 1, e)).astype(np.float32)


def pack_ue8m0(s: np.ndarray) -> np.ndarray:
    """Power-of-two fp32 scales [..., KB] -> packed UE8M0 words int32 [..., ceil(KB/4)]:
    the byte of K block 4w+i is byte i of word w (little-endian), and the byte
    is the scale's fp32 exponent field (2^-127 .. 2^127 -> 0 .. 254).  Padding
    bytes past KB hold 255 (the E8M0 NaN code), so reading one shows up."""
    s = np.ascontiguousarray(s, dtype=np.float32)
    lead = s.shape[:-1]
    s = s.reshape(-1, s.shape[-1])
    r, kb = s.shape
    m, _ = np.frexp(s.astype(np.float64))
    assert np.all(m == 0.5) and np.all(s > 0), "scales must be positive powers of two"
    assert np.all(s >= np.float32(2.0 ** -127)), "below the UE8M0 range"
    kw = (kb + 3) // 4
    raw = np.full((r, 4 * kw), 255, np.uint8)
    raw[:, :kb] = ((s.view(np.uint32) >> 23) & 0xFF).astype(np.uint8)
    return np.frombuffer(raw.tobytes(), dtype="<i4").reshape(*lead, kw).astype(np.int32)


def quantize_1x128(x: np.ndarray, pow2: bool = False) -> tuple[np.ndarray, np.ndarray]:
    """x fp32 [R, K] (K % 128 == 0) -> (q uint8 [R, K], s fp32 [R, K/128]).

    One scale per row and 128-wide K group, as the activation operand of the
    pages' usage example ([M, K] with [M, K//128] scales).  pow2: the scale is
    rounded up to a power of two (UE8M0 scales).
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    r, k = x.shape
    assert k % BLOCK_K == 0, "K must be a multiple of 128"
    g = x.reshape(r, k // BLOCK_K, BLOCK_K)
    amax = np.abs(g).max(axis=2)
    s = (amax / np.float32(E4M3_MAX)).astype(np.float32)
    s[amax == 0] = np.float32(1.0)
    if pow2:
        s = _pow2_ceil(s)
    y = np.clip(g / s[:, :, None], -E4M3_MAX, E4M3_MAX).astype(np.float32)
    return _encode_e4m3(y.reshape(r, k)), s


def quantize_128x128(x: np.ndarray, pow2: bool = False) -> tuple[np.ndarray, np.ndarray]:
    """x fp32 [N, K] -> (q uint8 [N, K], s fp32 [ceil(N/128), K/128]).

    One scale per 128x128 block, the last row block clipped to the rows that
    exist (the pages' example pairs N = 2112 with a [17, 56] scale tensor).
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    n, k = x.shape
    assert k % BLOCK_K == 0, "K must be a multiple of 128"
    nb = (n + BLOCK_K - 1) // BLOCK_K
    kb = k // BLOCK_K
    s = np.empty((nb, kb), dtype=np.float32)
    q = np.empty((n, k), dtype=np.uint8)
    for i in range(nb):
        blk = x[i * BLOCK_K:(i + 1) * BLOCK_K].reshape(-1, kb, BLOCK_K)
        amax = np.abs(blk).max(axis=(0, 2))
        si = (amax / np.float32(E4M3_MAX)).astype(np.float32)
        si[amax == 0] = np.float32(1.0)
        if pow2:
            si = _pow2_ceil(si)
        s[i] = si
        y = np.clip(blk / si[None, :, None], -E4M3_MAX, E4M3_MAX).astype(np.float32)
        q[i * BLOCK_K:(i + 1) * BLOCK_K] = _encode_e4m3(y.reshape(-1, k))
    return q, s


def _normal(rng: np.random.Generator, shape) -> np.ndarray:
    return rng.standard_normal(size=shape, dtype=np.float32)


@dataclass
class Dense:
    """Dense NT problem: A [M,K] + sa [M,K/128]; B [N,K] + sb [ceil(N/128),K/128]."""
    m: int
    n: int
    k: int
    a: np.ndarray
    sa: np.ndarray
    b: np.ndarray
    sb: np.ndarray


def make_dense(m: int, n: int, k: int, seed: int, pow2: bool = False) -> Dense:
    a, sa = quantize_1x128(_normal(_rng(seed, 0), (m, k)), pow2)
    b, sb = quantize_128x128(_normal(_rng(seed, 1), (n, k)), pow2)
    return Dense(m, n, k, a, sa, b, sb)


@dataclass
class DenseBf16:
    """Dense BF16 NT problem: A [M,K], B [N,K] as bf16 bit patterns (uint16)."""
    m: int
    n: int
    k: int
    a: np.ndarray
    b: np.ndarray


def _to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns via torch's CPU cast (round to nearest even)."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def make_dense_bf16(m: int, n: int, k: int, seed: int) -> DenseBf16:
    """N(0,1) operands rounded to bf16 (the same seeded streams as make_dense)."""
    return DenseBf16(m, n, k, _to_bf16_bits(_normal(_rng(seed, 0), (m, k))),
                     _to_bf16_bits(_normal(_rng(seed, 1), (n, k))))


def _expert_ids(g: int, rows_per_expert: int, seed: int, max_pad: int) -> np.ndarray:
    """Each expert's segment: its valid rows, then U{0..max_pad} padding rows (-1)."""
    pads = np.minimum(_rng(seed, 3).integers(0, max_pad + 1, size=g), rows_per_expert)
    ids = np.full(g * rows_per_expert, -1, dtype=np.int32)
    for e in range(g):
        ids[e * rows_per_expert:e * rows_per_expert + rows_per_expert - int(pads[e])] = e
    return ids


@dataclass
class GroupedBf16:
    """Grouped BF16 operands (bf16 bit patterns): contiguous a [M_total, K] with
    m_indices, or masked a [G, M_max, K] with masked_m; b [G, N, K]."""
    a: np.ndarray
    b: np.ndarray
    ctrl: np.ndarray


def make_contiguous_bf16(g: int, rows_per_expert: int, n: int, k: int, seed: int,
                         max_pad: int = 127) -> GroupedBf16:
    """N(0,1) values rounded to bf16; the contiguous layout of make_contiguous."""
    assert rows_per_expert % BLOCK_K == 0
    a = _to_bf16_bits(_normal(_rng(seed, 0), (g * rows_per_expert, k)))
    b = _to_bf16_bits(_normal(_rng(seed, 1), (g * n, k))).reshape(g, n, k)
    return GroupedBf16(a, b, _expert_ids(g, rows_per_expert, seed, max_pad))


def make_masked_bf16(g: int, m_max: int, n: int, k: int, seed: int, masked_m) -> GroupedBf16:
    a = _to_bf16_bits(_normal(_rng(seed, 0), (g * m_max, k))).reshape(g, m_max, k)
    b = _to_bf16_bits(_normal(_rng(seed, 1), (g * n, k))).reshape(g, n, k)
    return GroupedBf16(a, b, np.asarray(masked_m, dtype=np.int32))


def _grouped_rhs(g: int, n: int, k: int, seed: int, pow2: bool = False) -> tuple[np.ndarray, np.ndarray]:
    nb = (n + BLOCK_K - 1) // BLOCK_K
    b = np.empty((g, n, k), dtype=np.uint8)
    sb = np.empty((g, nb, k // BLOCK_K), dtype=np.float32)
    rng = _rng(seed, 1)
    for e in range(g):
        b[e], sb[e] = quantize_128x128(_normal(rng, (n, k)), pow2)
    return b, sb


@dataclass
class Contiguous:
    """MoE contiguous layout: rows of all experts stacked, one expert id per row.

    Each expert's segment is `rows_per_expert` rows (a multiple of 128): the
    first `valid[e]` rows carry id e, the rest are padding rows with id -1 that
    hold random A data (so wrongly computed padding is visible).
    """
    g: int
    m_total: int
    n: int
    k: int
    a: np.ndarray
    sa: np.ndarray
    b: np.ndarray
    sb: np.ndarray
    m_indices: np.ndarray
    valid: np.ndarray = field(default_factory=lambda: np.zeros(0, np.int64))


def make_contiguous(g: int, rows_per_expert: int, n: int, k: int, seed: int,
                    pad: bool = True, max_pad: int = 127, pow2: bool = False) -> Contiguous:
    """pow2: scales rounded up to powers of two (UE8M0-representable)."""
    assert rows_per_expert % BLOCK_K == 0
    m_total = g * rows_per_expert
    a, sa = quantize_1x128(_normal(_rng(seed, 0), (m_total, k)), pow2)
    b, sb = _grouped_rhs(g, n, k, seed, pow2)
    rng = _rng(seed, 3)
    pads = rng.integers(0, max_pad + 1, size=g) if pad else np.zeros(g, np.int64)
    pads = np.minimum(pads, rows_per_expert)
    ids = np.full(m_total, -1, dtype=np.int32)
    for e in range(g):
        v = rows_per_expert - int(pads[e])
        ids[e * rows_per_expert:e * rows_per_expert + v] = e
    return Contiguous(g, m_total, n, k, a, sa, b, sb, ids,
                      (rows_per_expert - pads).astype(np.int64))


@dataclass
class Masked:
    """MoE masked layout: A [G, M_max, K]; only rows < masked_m[g] are computed."""
    g: int
    m_max: int
    n: int
    k: int
    a: np.ndarray
    sa: np.ndarray
    b: np.ndarray
    sb: np.ndarray
    masked_m: np.ndarray


def make_masked(g: int, m_max: int, n: int, k: int, seed: int,
                lo: int = 64, hi: int = 192, masked_m=None, pow2: bool = False) -> Masked:
    """pow2: scales rounded up to powers of two (UE8M0-representable)."""
    a, sa = quantize_1x128(_normal(_rng(seed, 0), (g * m_max, k)), pow2)
    b, sb = _grouped_rhs(g, n, k, seed, pow2)
    if masked_m is None:
        masked_m = _rng(seed, 4).integers(lo, hi + 1, size=g)
    masked_m = np.asarray(masked_m, dtype=np.int32)
    return Masked(g, m_max, n, k, a.reshape(g, m_max, k), sa.reshape(g, m_max, k // BLOCK_K),
                  b, sb, masked_m)


@dataclass
class Wgrad:
    """Weight-gradient NT problem: both operands token-contiguous with 1x128 scales.

    A [M, T] + sa [M, T/128], B [N, T] + sb [N, T/128], D0 fp32 [G?, M, N].
    `ks` lists the token count of each group (one group for the dense case).
    """
    m: int
    n: int
    ks: list
    a: np.ndarray
    sa: np.ndarray
    b: np.ndarray
    sb: np.ndarray
    d0: np.ndarray


def make_wgrad(m: int, n: int, ks, seed: int) -> Wgrad:
    ks = [int(x) for x in ks]
    t = sum(ks)
    a, sa = quantize_1x128(_normal(_rng(seed, 0), (m, t)))
    b, sb = quantize_1x128(_normal(_rng(seed, 1), (n, t)))
    d0 = _normal(_rng(seed, 2), (len(ks), m, n))
    return Wgrad(m, n, ks, a, sa, b, sb, d0)


def _small_int_codes(rng: np.random.Generator, shape, top: int) -> np.ndarray:
    """e4m3 bytes of uniform integers in [-top, top] (exact in e4m3 for top <= 16)."""
    return _encode_e4m3(rng.integers(-top, top + 1, size=shape).astype(np.float32))


def _pow2_scales(rng: np.random.Generator, shape, lo: int, hi: int) -> np.ndarray:
    """fp32 scales 2^-e with e uniform in [lo, hi]."""
    return np.ldexp(np.float32(1.0), -rng.integers(lo, hi + 1, size=shape)).astype(np.float32)


def make_contiguous_exact(g: int, rows_per_expert: int, n: int, k: int, seed: int,
                          max_pad: int = 127, rows_expo=(2, 7), cols_expo=(2, 3)) -> Contiguous:
    """A contiguous problem whose every output is exactly representable in fp32.

    A and B hold small integers (|a| <= 4, |b| <= 4) and every scale is a power
    of two (sa = 2^-e per row and K block with e in `rows_expo`, sb = 2^-e per
    128x128 block with e in `cols_expo`), so each output is a multiple of
    2^-(max e sum) of modest size: any fp32 accumulation order gives it
    exactly and its bf16 rounding is unique.  With the default exponents and
    K <= 16384 the outputs are O(1) (|C| < 2^5)."""
    assert rows_per_expert % BLOCK_K == 0 and k % BLOCK_K == 0
    m_total = g * rows_per_expert
    nb, kb = (n + BLOCK_K - 1) // BLOCK_K, k // BLOCK_K
    a = _small_int_codes(_rng(seed, 0), (m_total, k), 4)
    sa = _pow2_scales(_rng(seed, 5), (m_total, kb), *rows_expo)
    b = _small_int_codes(_rng(seed, 1), (g, n, k), 4)
    sb = _pow2_scales(_rng(seed, 6), (g, nb, kb), *cols_expo)
    rng = _rng(seed, 3)
    pads = np.minimum(rng.integers(0, max_pad + 1, size=g), rows_per_expert)
    ids = np.full(m_total, -1, dtype=np.int32)
    for e in range(g):
        v = rows_per_expert - int(pads[e])
        ids[e * rows_per_expert:e * rows_per_expert + v] = e
    return Contiguous(g, m_total, n, k, a, sa, b, sb, ids, (rows_per_expert - pads).astype(np.int64))
