"""The C-ABI library on the CPU: it loads, exports every entry point that
include/dg.h declares, rejects bad arguments before touching the GPU, and its
tile heuristic obeys its invariants.  No compute call runs here."""
from __future__ import annotations

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dg.h")
LIB = os.path.join(ROOT, "moe_grouped_gemm_x128_amd", "libdg_mi355x.so")

INVALID, UNSUPPORTED, SUCCESS = 1, 2, 0


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        # run build.py as a script: importing it as a submodule would run the
        # package __init__, which refuses to load an unbuilt library
        import subprocess
        import sys
        subprocess.run([sys.executable, os.path.join(ROOT, "moe_grouped_gemm_x128_amd", "build.py")],
                       check=True)
    L = ctypes.CDLL(LIB)
    vp, i = ctypes.c_void_p, ctypes.c_int
    L.dg_gemm_fp8_nt.argtypes = [vp, vp, vp, vp, vp, i, i, i, vp]
    L.dg_grouped_fp8_contiguous.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, vp]
    L.dg_grouped_fp8_masked.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, vp]
    L.dg_wgrad_fp8_nt.argtypes = [vp, vp, vp, vp, vp, i, i, i, vp]
    L.dg_k_grouped_wgrad_fp8_nt.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, vp]
    L.dg_status_string.restype = ctypes.c_char_p
    return L


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:dg_status|const char\*|int)\s+(dg_\w+)\s*\(", text, re.M)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for f in ("dg_gemm_fp8_nt", "dg_grouped_fp8_contiguous", "dg_grouped_fp8_masked",
              "dg_wgrad_fp8_nt", "dg_k_grouped_wgrad_fp8_nt", "dg_status_string",
              "dg_select_config", "dg_version"):
        assert f in names


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_library_exports_nothing_but_c_symbols():
    """Every exported dg_ symbol is declared in the header (extern "C", unmangled)."""
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", LIB], capture_output=True, text=True).stdout
    exported = sorted({ln.split()[-1] for ln in out.splitlines() if " T dg_" in ln})
    assert exported == declared_functions()


def test_status_strings(lib):
    for s in range(4):
        assert len(lib.dg_status_string(s)) > 3
    assert lib.dg_status_string(99) == b"unknown status"
    assert lib.dg_version() >= 100


# Fake device addresses: validation must reject before any dereference or HIP call.
A16 = 0x10000
MIS = 0x10001


def test_dense_argument_errors(lib):
    f = lib.dg_gemm_fp8_nt
    assert f(None, A16, A16, A16, A16, 1, 1, 128, None) == INVALID
    assert f(A16, A16, A16, A16, None, 1, 1, 128, None) == INVALID
    assert f(A16, A16, A16, A16, A16, 0, 1, 128, None) == INVALID
    assert f(A16, A16, A16, A16, A16, 1, -5, 128, None) == INVALID
    assert f(A16, A16, A16, A16, A16, 1, 1, 0, None) == INVALID
    assert f(A16, A16, A16, A16, A16, 1, 1, 100, None) == UNSUPPORTED   # K % 128
    assert f(MIS, A16, A16, A16, A16, 1, 1, 128, None) == UNSUPPORTED   # a not 16B aligned
    assert f(A16, A16, A16 + 8, A16, A16, 1, 1, 128, None) == UNSUPPORTED
    assert f(A16, A16 + 2, A16, A16, A16, 1, 1, 128, None) == UNSUPPORTED  # scale alignment
    assert f(A16, A16, A16, A16, MIS, 1, 1, 128, None) == UNSUPPORTED   # bf16 alignment


def test_grouped_argument_errors(lib):
    c = lib.dg_grouped_fp8_contiguous
    assert c(A16, A16, A16, A16, A16, None, 128, 8, 128, 2, None) == INVALID
    assert c(A16, A16, A16, A16, A16, A16, 128, 8, 128, 0, None) == INVALID
    assert c(A16, A16, A16, A16, A16, A16, 100, 8, 128, 2, None) == UNSUPPORTED  # M_total % 128
    assert c(A16, A16, A16, A16, A16, A16, 128, 8, 384 + 64, 2, None) == UNSUPPORTED
    assert c(A16, A16, A16, A16, A16, A16 + 2, 128, 8, 128, 2, None) == UNSUPPORTED
    m = lib.dg_grouped_fp8_masked
    assert m(A16, A16, A16, A16, A16, None, 2, 256, 8, 128, None) == INVALID
    assert m(A16, A16, A16, A16, A16, A16, 0, 256, 8, 128, None) == INVALID
    assert m(A16, A16, A16, A16, A16, A16, 2, 0, 8, 128, None) == INVALID
    assert m(A16, A16, A16, A16, A16, A16, 2, 256, 8, 200, None) == UNSUPPORTED


def test_fused_swiglu_argument_errors(lib):
    f = lib.dg_grouped_fp8_contiguous_swiglu
    f.argtypes = [ctypes.c_void_p] * 7 + [ctypes.c_int] * 4 + [ctypes.c_void_p]
    ok = (A16, A16, A16, A16, A16, A16, A16)
    for i in range(7):
        args = list(ok)
        args[i] = None
        assert f(*args, 256, 512, 128, 2, None) == INVALID, i
    assert f(*ok, 0, 512, 128, 2, None) == INVALID
    assert f(*ok, 256, 512, 128, 0, None) == INVALID
    assert f(*ok, 256, 384, 128, 2, None) == UNSUPPORTED      # N % 256: I not a multiple of 128
    assert f(*ok, 200, 512, 128, 2, None) == UNSUPPORTED      # M_total % 128
    assert f(*ok, 256, 512, 200, 2, None) == UNSUPPORTED      # K % 128
    assert f(*ok, 256, 1 << 20, 1 << 13, 2, None) == UNSUPPORTED  # one B range past 32 bits
    assert f(MIS, A16, A16, A16, A16, A16, A16, 256, 512, 128, 2, None) == UNSUPPORTED
    assert f(A16, A16, A16, A16, A16 + 2, A16, A16, 256, 512, 128, 2, None) == UNSUPPORTED  # q alignment
    assert f(A16, A16, A16, A16, A16, A16 + 2, A16, 256, 512, 128, 2, None) == UNSUPPORTED  # s alignment


def test_fused_swiglu_plan(lib):
    """One tile: 256 rows x (128 gate + 128 up columns) on 2x4 waves, never split."""
    c = _cfg(lib, 7, 65536, 4096, 7168)
    assert (c["block_m"], c["block_n"], c["waves_m"], c["waves_n"]) == (256, 256, 2, 4)
    assert c["tiles"] == (65536 // 256) * (4096 // 256) and c["k_splits"] == 1


def test_bf16_argument_errors(lib):
    f = lib.dg_gemm_bf16_nt
    f.argtypes = [ctypes.c_void_p] * 3 + [ctypes.c_int] * 3 + [ctypes.c_void_p]
    assert f(None, A16, A16, 1, 1, 64, None) == INVALID
    assert f(A16, A16, None, 1, 1, 64, None) == INVALID
    assert f(A16, A16, A16, 1, 0, 64, None) == INVALID
    assert f(A16, A16, A16, 1, 1, 96, None) == UNSUPPORTED    # K % 64
    assert f(A16, A16, A16, 1, 1, 1 << 23, None) == UNSUPPORTED
    assert f(MIS, A16, A16, 1, 1, 64, None) == UNSUPPORTED    # a alignment
    assert f(A16, A16, MIS, 1, 1, 64, None) == UNSUPPORTED    # c alignment


def test_ue8m0_argument_errors(lib):
    f = lib.dg_gemm_fp8_nt_ue8m0
    f.argtypes = [ctypes.c_void_p] * 5 + [ctypes.c_int] * 3 + [ctypes.c_void_p]
    assert f(None, A16, A16, A16, A16, 1, 1, 128, None) == INVALID
    assert f(A16, A16, A16, A16, None, 1, 1, 128, None) == INVALID
    assert f(A16, A16, A16, A16, A16, 0, 1, 128, None) == INVALID
    assert f(A16, A16, A16, A16, A16, 1, 1, 100, None) == UNSUPPORTED   # K % 128
    assert f(MIS, A16, A16, A16, A16, 1, 1, 128, None) == UNSUPPORTED   # a alignment
    assert f(A16, A16 + 2, A16, A16, A16, 1, 1, 128, None) == UNSUPPORTED


def test_ue8m0_packed_argument_errors(lib):
    f = lib.dg_gemm_fp8_nt_ue8m0_packed
    f.argtypes = [ctypes.c_void_p] * 5 + [ctypes.c_int] * 3 + [ctypes.c_void_p]
    assert f(None, A16, A16, A16, A16, 1, 1, 128, None) == INVALID
    assert f(A16, None, A16, A16, A16, 1, 1, 128, None) == INVALID
    assert f(A16, A16, A16, None, A16, 1, 1, 128, None) == INVALID
    assert f(A16, A16, A16, A16, A16, 1, -1, 128, None) == INVALID
    assert f(A16, A16, A16, A16, A16, 1, 1, 640 + 64, None) == UNSUPPORTED   # K % 128
    assert f(A16, A16 + 2, A16, A16, A16, 1, 1, 128, None) == UNSUPPORTED    # sa words
    assert f(A16, A16, A16, A16 + 1, A16, 1, 1, 128, None) == UNSUPPORTED    # sb words
    assert f(A16, A16, A16 + 8, A16, A16, 1, 1, 128, None) == UNSUPPORTED    # b alignment


def test_grouped_bf16_argument_errors(lib):
    vp, i = ctypes.c_void_p, ctypes.c_int
    fc = lib.dg_grouped_bf16_contiguous
    fc.argtypes = [vp] * 4 + [i] * 4 + [vp]
    assert fc(A16, A16, A16, None, 256, 512, 128, 2, None) == INVALID     # m_indices
    assert fc(A16, A16, A16, A16, 256, 512, 96, 2, None) == UNSUPPORTED   # K % 64
    assert fc(A16, A16, A16, A16, 200, 512, 128, 2, None) == UNSUPPORTED  # M_total % 128
    assert fc(A16, A16 + 8, A16, A16, 256, 512, 128, 2, None) == UNSUPPORTED
    fm = lib.dg_grouped_bf16_masked
    fm.argtypes = [vp] * 4 + [i] * 4 + [vp]
    assert fm(A16, A16, A16, None, 2, 256, 512, 128, None) == INVALID      # masked_m
    assert fm(A16, A16, A16, A16, 0, 256, 512, 128, None) == INVALID       # G
    assert fm(A16, A16, A16, A16, 2, 256, 512, 1 << 23, None) == UNSUPPORTED
    assert fm(A16, A16, MIS, A16, 2, 256, 512, 128, None) == UNSUPPORTED   # c alignment


def test_grouped_ue8m0_packed_argument_errors(lib):
    vp, i = ctypes.c_void_p, ctypes.c_int
    fc = lib.dg_grouped_fp8_contiguous_ue8m0_packed
    fc.argtypes = [vp] * 6 + [i] * 4 + [vp]
    assert fc(A16, A16, A16, A16, A16, None, 256, 512, 128, 2, None) == INVALID   # m_indices
    assert fc(A16, A16, A16, A16, A16, A16, 256, 512, 128, 0, None) == INVALID    # G
    assert fc(A16, A16, A16, A16, A16, A16, 200, 512, 128, 2, None) == UNSUPPORTED  # M_total % 128
    assert fc(A16, A16 + 2, A16, A16, A16, A16, 256, 512, 128, 2, None) == UNSUPPORTED
    fm = lib.dg_grouped_fp8_masked_ue8m0_packed
    fm.argtypes = [vp] * 6 + [i] * 4 + [vp]
    assert fm(A16, A16, A16, A16, A16, None, 2, 256, 512, 128, None) == INVALID    # masked_m
    assert fm(A16, A16, A16, A16, A16, A16, 2, 0, 512, 128, None) == INVALID       # M_max
    assert fm(A16, A16, A16, A16, A16, A16, 2, 256, 512, 200, None) == UNSUPPORTED  # K % 128
    assert fm(A16, A16, A16, A16 + 1, A16, A16, 2, 256, 512, 128, None) == UNSUPPORTED


def test_quantizer_argument_errors(lib):
    vp, i = ctypes.c_void_p, ctypes.c_int
    for name in ("dg_quantize_fp8_1x128", "dg_quantize_fp8_128x128", "dg_quantize_fp8_1x128_transposed",
                 "dg_quantize_fp8_1x128_ue8m0", "dg_quantize_fp8_128x128_ue8m0"):
        f = getattr(lib, name)
        f.argtypes = [vp, vp, vp, i, i, vp]
        assert f(None, A16, A16, 128, 128, None) == INVALID, name
        assert f(A16, None, A16, 128, 128, None) == INVALID, name
        assert f(A16, A16, None, 128, 128, None) == INVALID, name
        assert f(A16, A16, A16, 0, 128, None) == INVALID, name
        assert f(A16, A16, A16, 128, -1, None) == INVALID, name
        assert f(A16 + 4, A16, A16, 128, 128, None) == UNSUPPORTED, name   # x not 16-byte aligned
        assert f(A16, A16, A16 + 2, 128, 128, None) == UNSUPPORTED, name   # scale alignment
    q1 = lib.dg_quantize_fp8_1x128
    assert q1(A16, A16, A16, 128, 100, None) == UNSUPPORTED               # K % 128
    assert q1(A16, A16 + 2, A16, 128, 128, None) == UNSUPPORTED           # q alignment
    qb = lib.dg_quantize_fp8_128x128
    assert qb(A16, A16, A16, 100, 200, None) == UNSUPPORTED
    qt = lib.dg_quantize_fp8_1x128_transposed
    assert qt(A16, A16, A16, 100, 128, None) == UNSUPPORTED               # T % 128
    assert qt(A16, A16, A16, 128, 130, None) == UNSUPPORTED               # F % 4
    assert qt(A16, A16 + 4, A16, 128, 128, None) == UNSUPPORTED           # q 16-byte alignment


def test_swiglu_quantizer_argument_errors(lib):
    vp, i = ctypes.c_void_p, ctypes.c_int
    f = lib.dg_swiglu_quantize_fp8_1x128
    f.argtypes = [vp, vp, vp, i, i, vp]
    assert f(None, A16, A16, 4, 128, None) == INVALID
    assert f(A16, None, A16, 4, 128, None) == INVALID
    assert f(A16, A16, None, 4, 128, None) == INVALID
    assert f(A16, A16, A16, 0, 128, None) == INVALID
    assert f(A16, A16, A16, 4, 0, None) == INVALID
    assert f(A16, A16, A16, 4, 192, None) == UNSUPPORTED                 # I % 128
    assert f(A16, A16, A16, 4, (1 << 30) + 128, None) == UNSUPPORTED     # 2I overflows an int
    assert f(A16 + 8, A16, A16, 4, 128, None) == UNSUPPORTED             # c 16-byte alignment
    assert f(A16, A16 + 4, A16, 4, 128, None) == UNSUPPORTED             # q 8-byte alignment
    assert f(A16, A16, A16 + 2, 4, 128, None) == UNSUPPORTED             # s alignment


def test_wgrad_argument_errors(lib):
    w = lib.dg_wgrad_fp8_nt
    assert w(A16, A16, A16, A16, None, 4, 4, 128, None) == INVALID
    assert w(A16, A16, A16, A16, A16, 4, 4, 96, None) == UNSUPPORTED
    assert w(A16, A16, A16, A16, A16 + 2, 4, 4, 128, None) == UNSUPPORTED
    kg = lib.dg_k_grouped_wgrad_fp8_nt
    ks = (ctypes.c_int32 * 3)(128, 256, 0)
    assert kg(A16, A16, A16, A16, A16, None, 3, 4, 4, None) == INVALID
    assert kg(A16, A16, A16, A16, A16, ks, 0, 4, 4, None) == INVALID
    assert kg(A16, A16, A16, A16, A16, ks, 257, 4, 4, None) == UNSUPPORTED
    bad = (ctypes.c_int32 * 2)(128, 100)
    assert kg(A16, A16, A16, A16, A16, bad, 2, 4, 4, None) == UNSUPPORTED
    neg = (ctypes.c_int32 * 2)(128, -128)
    assert kg(A16, A16, A16, A16, A16, neg, 2, 4, 4, None) == INVALID
    zero = (ctypes.c_int32 * 2)(0, 0)
    assert kg(A16, A16, A16, A16, A16, zero, 2, 4, 4, None) == SUCCESS  # nothing to do, nothing enqueued


# ------------------------------------------------------------- heuristic ---

def _cfg(lib, kind, m, n, k, g=1, cus=256):
    class Cfg(ctypes.Structure):
        _fields_ = [(f, ctypes.c_int) for f in ("block_m", "block_n", "waves_m", "waves_n", "tiles", "grid",
                                                "k_splits", "kernel")]
    c = Cfg()
    lib.dg_select_config.argtypes = [ctypes.c_int] * 6 + [ctypes.POINTER(Cfg)]
    st = lib.dg_select_config(kind, m, n, k, g, cus, ctypes.byref(c))
    assert st == SUCCESS
    return {f: getattr(c, f) for f, _ in Cfg._fields_}


SHAPES = [(0, m, n, k, 1) for m in (1, 64, 128, 4096)
          for (n, k) in [(2112, 7168), (24576, 1536), (32768, 512), (7168, 16384), (4096, 7168), (7168, 2048)]]
SHAPES += [(1, 32768, 4096, 7168, 4), (1, 65536, 7168, 2048, 8), (2, 256, 4096, 7168, 1),
           (2, 256, 7168, 2048, 16), (3, 7168, 2048, 4096, 1), (4, 7168, 2048, 10240, 4)]
SHAPES += [(5, m, 7168, 16384, 1) for m in (64, 4096)] + [(6, m, 7168, 8192, 1) for m in (64, 4096)]
SHAPES += [(8, 32768, 4096, 7168, 4), (9, 256, 4096, 7168, 1), (9, 256, 7168, 2048, 16)]
SHAPES += [(10, 32768, 4096, 7168, 4), (11, 256, 4096, 7168, 1), (11, 256, 7168, 2048, 16)]


@pytest.mark.parametrize("kind,m,n,k,g", SHAPES)
def test_heuristic_invariants(lib, kind, m, n, k, g):
    c = _cfg(lib, kind, m, n, k, g)
    assert c["waves_m"] * c["waves_n"] in (4, 8)
    assert c["block_m"] % (16 * c["waves_m"]) == 0 and c["block_n"] % (16 * c["waves_n"]) == 0
    groups = g if kind in (2, 4, 9, 11) else 1
    tiles = groups * -(-m // c["block_m"]) * -(-n // c["block_n"])
    assert c["tiles"] == tiles
    s = c["k_splits"]
    assert 1 <= s <= 16
    if kind not in (0, 2, 5, 6, 9, 11):
        assert s == 1  # split K only for the bf16-output dense and masked layouts
    kbs = k // 64 if kind in (6, 10, 11) else k // 128  # BF16: K blocks of 64 values (128 bytes)
    if s > 1:
        chunk = -(-kbs // s)
        assert -(-kbs // chunk) == s, "a split would be empty"
        assert chunk >= 4
    # one pass over the work items when they fit: the grid is the item count
    # rounded up to a multiple of 8 (no workgroup takes two items while others idle)
    work = tiles * s
    assert 1 <= c["grid"] <= -(-work // 8) * 8
    if work <= 256:
        assert c["grid"] >= work
    assert c["kernel"] == 0
    if c["grid"] > 8:
        assert c["grid"] % 8 == 0
    assert c["grid"] <= 2 * 256
    assert _cfg(lib, kind, m, n, k, g) == c  # deterministic


def test_masked_plan(lib):
    """Masked decode: the general kernel's tall tiles serve every page shape,
    long K is split until the CUs are covered, short K is not split."""
    for g in (1, 2, 4, 16):
        for n, k in ((4096, 7168), (7168, 2048)):
            c = _cfg(lib, 2, 256, n, k, g)
            assert c["kernel"] == 0 and c["block_m"] == 256
            if k == 2048:
                assert c["k_splits"] == 1
            elif c["tiles"] < 180:
                assert c["tiles"] * c["k_splits"] >= 256 and (k // 128) // c["k_splits"] >= 6
    assert _cfg(lib, 2, 256, 4096, 7168, 16)["block_n"] == 256
    # short K, one group: 32-column tiles fill the CUs without a split
    c = _cfg(lib, 2, 256, 7168, 2048, 1)
    assert (c["block_m"], c["block_n"], c["k_splits"]) == (256, 32, 1)


def test_power_of_two_kinds_plan_as_their_layout(lib):
    """The packed-UE8M0 grouped kinds take their fp32-scale kind's plan."""
    for (kind, base, m, n, k, g) in [(8, 1, 65536, 4096, 7168, 8), (8, 1, 32768, 7168, 2048, 4),
                                     (9, 2, 256, 4096, 7168, 1), (9, 2, 256, 4096, 7168, 16),
                                     (9, 2, 256, 7168, 2048, 4), (5, 0, 64, 2112, 7168, 1)]:
        assert _cfg(lib, kind, m, n, k, g) == _cfg(lib, base, m, n, k, g), (kind, m, n, k, g)


def test_split_k_planning(lib):
    """Few output tiles and a long K: split K four ways (with 64-column tiles
    when the 128-column ones are too few: fewer, larger items than CUs
    measured faster for M=64, N=2112, K=7168); many tiles: no split."""
    c = _cfg(lib, 0, 64, 2112, 7168)
    assert c["k_splits"] == 4 and (c["block_m"], c["block_n"]) == (64, 64) and c["tiles"] * c["k_splits"] >= 128
    c = _cfg(lib, 0, 64, 4096, 7168)
    assert c["k_splits"] == 4 and c["tiles"] * c["k_splits"] >= 256
    c = _cfg(lib, 2, 256, 4096, 7168, 1)
    assert c["k_splits"] > 1
    assert _cfg(lib, 0, 4096, 7168, 16384)["k_splits"] == 1
    assert _cfg(lib, 0, 64, 2112, 384)["k_splits"] == 1  # K too short to split
    assert _cfg(lib, 3, 64, 2112, 7168)["k_splits"] == 1  # fp32-accumulate layouts never split


def test_heuristic_rejects_bad_queries(lib):
    c = ctypes.c_int * 8
    out = c()
    lib.dg_select_config.argtypes = [ctypes.c_int] * 6 + [ctypes.c_void_p]
    assert lib.dg_select_config(12, 1, 1, 128, 1, 256, ctypes.addressof(out)) == INVALID
    assert lib.dg_select_config(-1, 1, 1, 128, 1, 256, ctypes.addressof(out)) == INVALID
    # the fused SwiGLU kind needs N % 256 == 0 and M % 128 == 0
    assert lib.dg_select_config(7, 128, 384, 128, 1, 256, ctypes.addressof(out)) == UNSUPPORTED
    assert lib.dg_select_config(7, 100, 512, 128, 1, 256, ctypes.addressof(out)) == UNSUPPORTED
    assert lib.dg_select_config(0, 0, 1, 128, 1, 256, ctypes.addressof(out)) == INVALID
    assert lib.dg_select_config(0, 1, 1, 128, 1, 256, None) == INVALID


def test_python_binding_rejects_cpu_tensors_and_bad_shapes():
    import torch
    import moe_grouped_gemm_x128_amd as dg
    a = torch.zeros(4, 128, dtype=torch.uint8)
    sa = torch.ones(4, 1)
    b = torch.zeros(8, 128, dtype=torch.uint8)
    sb = torch.ones(1, 1)
    c = torch.empty(4, 8, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        dg.dg_gemm_fp8_nt(a, sa, b, sb, c)               # host tensors
    with pytest.raises(ValueError):
        dg.dg_gemm_fp8_nt(a, torch.ones(4, 2), b, sb, c)  # scale shape
    with pytest.raises(TypeError):
        dg.dg_gemm_fp8_nt(a, sa.double(), b, sb, c)
    assert dg.select_config(dg.KIND_DENSE, 4096, 7168, 16384)["tiles"] > 0
    # SwiGLU input of odd width: the gate / up halves are undefined
    odd = torch.empty(4, 257, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        dg.dg_swiglu_quantize_fp8_1x128(odd, torch.empty(4, 128, dtype=torch.uint8).view(torch.float8_e4m3fn),
                                        torch.empty(4, 1))
    with pytest.raises(ValueError):
        dg.swiglu_quantize_fp8_1x128(odd)
