"""Pins for the oracle's packed-UE8M0 step (oracle.unpack_ue8m0 and
oracle.gemm_fp8_nt_ue8m0_packed), on the CPU, each against something other
than the unpacking arithmetic itself:

  * printed values of the E8M0 exponent code: bias 127, 0 -> 2^-127 (the fp32
    subnormal 0x00400000), 1 -> the smallest normal fp32, 127 -> 1, 254 ->
    2^127, 255 -> NaN, written here as the fp32 bit patterns numpy decodes;
  * byte order: words built from byte strings by Python's own little-endian
    int.from_bytes, so byte i of word w is K block 4w + i;
  * the IEEE route: a positive power-of-two fp32 scale's exponent field is its
    E8M0 byte, so packing the fields of random scales and unpacking gives the
    scales back bit for bit;
  * padding bytes past the last K block are ignored;
  * the packed GEMM is the dense oracle on the same scales given as fp32.
Plausible mistakes in an unpacker (big-endian bytes, bias 128, a dropped NaN
code, a word index of kb // 8) must each fail one of these pins."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from harness import inputs


def f32_bits(*words: int) -> np.ndarray:
    return np.array(words, np.uint32).view(np.float32)


def word_of(b0: int, b1: int, b2: int, b3: int) -> int:
    v = int.from_bytes(bytes([b0, b1, b2, b3]), "little")
    return v - (1 << 32) if v >= 1 << 31 else v


def pin_codes(unpack) -> bool:
    """Printed code values (fp32 bit patterns), one code per K block."""
    # codes 0, 1, 126, 127, 128, 200, 254
    want = f32_bits(0x00400000, 0x00800000, 0x3F000000, 0x3F800000, 0x40000000, 0x64000000, 0x7F000000)
    words = np.array([[word_of(0, 1, 126, 127), word_of(128, 200, 254, 7)]], np.int32)
    got = unpack(words, 7)[0]
    nan = unpack(np.array([[word_of(255, 127, 255, 127)]], np.int32), 4)[0]
    return (np.array_equal(got.view(np.uint32), want.view(np.uint32)) and bool(np.isnan(nan[0]))
            and bool(np.isnan(nan[2])) and nan[1] == 1.0 and nan[3] == 1.0)


def pin_byte_order(unpack) -> bool:
    """K block 4w+i is byte i of word w: distinct codes in every byte."""
    raw = np.arange(100, 124, dtype=np.uint8).reshape(2, 12)    # 2 rows x 12 K blocks
    words = np.array([[word_of(*raw[r, 4 * w:4 * w + 4]) for w in range(3)] for r in range(2)], np.int32)
    got = unpack(words, 12)
    want = np.ldexp(np.float32(1.0), raw.astype(np.int32) - 127)
    return np.array_equal(got, want)


def pin_ieee_round_trip(unpack) -> bool:
    """Random power-of-two fp32 scales: their exponent fields, packed, unpack to themselves."""
    rng = np.random.default_rng(31)
    for kb in (1, 3, 4, 5, 56, 128):
        s = np.ldexp(np.float32(1.0), rng.integers(-127, 128, (9, kb))).astype(np.float32)
        if not np.array_equal(unpack(inputs.pack_ue8m0(s), kb).view(np.uint32), s.view(np.uint32)):
            return False
    return True


def pin_padding_ignored(unpack) -> bool:
    """Bytes past the last K block hold anything, the NaN code included."""
    base = np.array([[word_of(127, 128, 129, 255)]], np.int32)
    other = np.array([[word_of(127, 128, 129, 3)]], np.int32)
    a, b = unpack(base, 3), unpack(other, 3)
    return np.array_equal(a, b) and not np.any(np.isnan(a))


PINS = [pin_codes, pin_byte_order, pin_ieee_round_trip, pin_padding_ignored]


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_unpack_pins(pin):
    assert pin(oracle.unpack_ue8m0)


def test_packed_gemm_is_the_dense_oracle():
    """K = 640 (5 K blocks: two words, the last one padded) and ragged M, N."""
    d = inputs.make_dense(37, 150, 640, seed=inputs.SEED_BASE + 60, pow2=True)
    c1, x1 = oracle.gemm_fp8_nt_ue8m0_packed(d.a, inputs.pack_ue8m0(d.sa), d.b, inputs.pack_ue8m0(d.sb))
    c0, x0 = oracle.gemm_fp8_nt(d.a, d.sa, d.b, d.sb)
    assert np.array_equal(c1, c0) and np.array_equal(x1, x0)


def test_packer_layout():
    """The input packer's words, read back as bytes, are the exponent fields in
    K-block order, then 255s."""
    s = np.ldexp(np.float32(1.0), np.array([[-127, 0, 5, 127, -1]])).astype(np.float32)
    raw = np.frombuffer(inputs.pack_ue8m0(s).astype("<i4").tobytes(), np.uint8)
    assert raw.tolist() == [0, 127, 132, 254, 126, 255, 255, 255]


# ---- planted mistakes: each must fail at least one pin -------------------------

def _mutant(order="little", bias=127, nan=True, per_word=4):
    def unpack(words, kblocks):
        w = np.ascontiguousarray(words).astype(np.int64) & 0xFFFFFFFF
        out = np.empty((w.shape[0], kblocks), np.float64)
        for kb in range(kblocks):
            i = kb % 4 if order == "little" else 3 - kb % 4
            e = (w[:, min(kb // per_word, w.shape[1] - 1)] >> (8 * i)) & 0xFF
            v = np.ldexp(1.0, (e - bias).astype(np.int32))
            out[:, kb] = np.where(e == 255, np.nan, v) if nan else v
        with np.errstate(over="ignore"):   # bias 128 can give 2^128: inf in fp32
            return out.astype(np.float32)
    return unpack


@pytest.mark.parametrize("mutant", [dict(order="big"), dict(bias=128), dict(nan=False), dict(per_word=8)],
                         ids=["big_endian", "bias_128", "no_nan_code", "eight_per_word"])
def test_planted_mistakes_fail_a_pin(mutant):
    bad = _mutant(**mutant)
    assert not all(pin(bad) for pin in PINS), f"no pin catches {mutant}"
    assert all(pin(_mutant()) for pin in PINS), "the unmutated rewrite must pass every pin"


def test_grouped_packed_oracles_are_the_grouped_oracles():
    """Scales of any rank unpack along their last axis; the grouped packed
    oracles are the grouped oracles on the unpacked scales."""
    from tests.parity import SENTINEL_BF16
    x = inputs.make_contiguous(3, 256, 140, 640, seed=inputs.SEED_BASE + 66, pow2=True)
    assert inputs.pack_ue8m0(x.sb).shape == (3, 2, 2)
    assert np.array_equal(oracle.unpack_ue8m0(inputs.pack_ue8m0(x.sb), 5), x.sb)
    init = np.full((x.m_total, x.n), SENTINEL_BF16, np.uint16)
    got = oracle.grouped_contiguous_ue8m0_packed(x.a, inputs.pack_ue8m0(x.sa), x.b, inputs.pack_ue8m0(x.sb),
                                                 x.m_indices, init)
    want = oracle.grouped_contiguous(x.a, x.sa, x.b, x.sb, x.m_indices, init)
    assert np.array_equal(got[0], want[0]) and np.array_equal(got[1], want[1], equal_nan=True)
    mm = np.array([0, 5, 70], np.int32)
    y = inputs.make_masked(3, 70, 140, 640, seed=inputs.SEED_BASE + 67, masked_m=mm, pow2=True)
    init = np.full((3, 70, 140), SENTINEL_BF16, np.uint16)
    got = oracle.grouped_masked_ue8m0_packed(y.a, inputs.pack_ue8m0(y.sa), y.b, inputs.pack_ue8m0(y.sb), mm, init)
    want = oracle.grouped_masked(y.a, y.sa, y.b, y.sb, mm, init)
    assert np.array_equal(got[0], want[0])
