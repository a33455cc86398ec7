"""Python binding of the MI355X FP8 fine-grained-scaled NT GEMM library.

Argument marshalling only: every function below checks tensor dtypes, shapes
and devices, then calls the C ABI (include/dg.h) of libdg_mi355x.so with raw
device pointers and the current HIP stream.  All arithmetic runs in the HIP
kernels; there is no CPU path.  If the library has not been built the import
fails loudly (build it with `python moe_grouped_gemm_x128_amd/build.py`).

The C-named functions mirror the C entry points one to one.  The
`*_fp8_fp8_*` names follow the call style of the DeepGEMM pages' usage example
(operands passed as (fp8 tensor, fp32 scale tensor) tuples, output tensor
preallocated by the caller).
"""
from __future__ import annotations

import ctypes
import os

import torch  # loads torch's HIP runtime first, so the library binds to it

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdg_mi355x.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build the HIP library first "
        "(python moe_grouped_gemm_x128_amd/build.py); there is no fallback path")

_lib = ctypes.CDLL(LIB_PATH)

_vp, _i32 = ctypes.c_void_p, ctypes.c_int
_lib.dg_gemm_fp8_nt.argtypes = [_vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _vp]
_lib.dg_grouped_fp8_contiguous.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _vp]
_lib.dg_grouped_fp8_contiguous_swiglu.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _vp]
_lib.dg_grouped_fp8_masked.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _vp]
_lib.dg_grouped_fp8_masked_noalloc.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _vp]
_lib.dg_wgrad_fp8_nt.argtypes = [_vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _vp]
_lib.dg_k_grouped_wgrad_fp8_nt.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _vp]
_lib.dg_gemm_fp8_nt_ue8m0.argtypes = [_vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _vp]
_lib.dg_gemm_fp8_nt_ue8m0_packed.argtypes = [_vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _vp]
_lib.dg_grouped_fp8_contiguous_ue8m0_packed.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _vp]
_lib.dg_grouped_fp8_masked_ue8m0_packed.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _vp]
_lib.dg_gemm_bf16_nt.argtypes = [_vp, _vp, _vp, _i32, _i32, _i32, _vp]
_lib.dg_grouped_bf16_contiguous.argtypes = [_vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _vp]
_lib.dg_grouped_bf16_masked.argtypes = [_vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _vp]
_lib.dg_quantize_fp8_1x128.argtypes = [_vp, _vp, _vp, _i32, _i32, _vp]
_lib.dg_quantize_fp8_128x128.argtypes = [_vp, _vp, _vp, _i32, _i32, _vp]
_lib.dg_quantize_fp8_1x128_transposed.argtypes = [_vp, _vp, _vp, _i32, _i32, _vp]
_lib.dg_quantize_fp8_1x128_ue8m0.argtypes = [_vp, _vp, _vp, _i32, _i32, _vp]
_lib.dg_quantize_fp8_128x128_ue8m0.argtypes = [_vp, _vp, _vp, _i32, _i32, _vp]
_lib.dg_swiglu_quantize_fp8_1x128.argtypes = [_vp, _vp, _vp, _i32, _i32, _vp]
for _f in ("dg_gemm_fp8_nt", "dg_grouped_fp8_contiguous", "dg_grouped_fp8_contiguous_swiglu", "dg_grouped_fp8_masked", "dg_grouped_fp8_masked_noalloc",
           "dg_wgrad_fp8_nt", "dg_k_grouped_wgrad_fp8_nt", "dg_gemm_fp8_nt_ue8m0", "dg_gemm_fp8_nt_ue8m0_packed", "dg_grouped_fp8_contiguous_ue8m0_packed",
           "dg_grouped_fp8_masked_ue8m0_packed", "dg_gemm_bf16_nt", "dg_grouped_bf16_contiguous", "dg_grouped_bf16_masked", "dg_quantize_fp8_1x128",
           "dg_quantize_fp8_128x128", "dg_quantize_fp8_1x128_transposed", "dg_swiglu_quantize_fp8_1x128",
           "dg_quantize_fp8_1x128_ue8m0", "dg_quantize_fp8_128x128_ue8m0"):
    getattr(_lib, _f).restype = ctypes.c_int
_lib.dg_status_string.argtypes = [ctypes.c_int]
_lib.dg_status_string.restype = ctypes.c_char_p
_lib.dg_version.restype = ctypes.c_int


class TileConfig(ctypes.Structure):
    _fields_ = [("block_m", ctypes.c_int), ("block_n", ctypes.c_int), ("waves_m", ctypes.c_int),
                ("waves_n", ctypes.c_int), ("tiles", ctypes.c_int), ("grid", ctypes.c_int),
                ("k_splits", ctypes.c_int), ("kernel", ctypes.c_int)]


_lib.dg_select_config.argtypes = [_i32, _i32, _i32, _i32, _i32, _i32, ctypes.POINTER(TileConfig)]
_lib.dg_select_config.restype = ctypes.c_int

(KIND_DENSE, KIND_CONTIGUOUS, KIND_MASKED, KIND_WGRAD, KIND_K_GROUPED_WGRAD, KIND_DENSE_POW2, KIND_BF16,
 KIND_CONTIGUOUS_SWIGLU, KIND_CONTIGUOUS_POW2, KIND_MASKED_POW2, KIND_CONTIGUOUS_BF16, KIND_MASKED_BF16) = range(12)
FP8 = torch.float8_e4m3fn


class DGError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = _lib.dg_status_string(status).decode()
        super().__init__(f"{where}: status {status} ({msg})")


def _check(status: int, where: str):
    if status != 0:
        raise DGError(status, where)


# The current stream's raw handle without building a torch Stream object
# (a few microseconds per call otherwise, which small GEMMs would feel).
_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream(t: torch.Tensor):
    if _raw_stream is not None:
        return _raw_stream(t.get_device())
    return torch.cuda.current_stream(t.device).cuda_stream


def _ptr(t):
    return t.data_ptr()


def _dev(*ts):
    if not ts[0].is_cuda:
        raise ValueError("tensors must live on the GPU")
    dev = ts[0].get_device()
    for t in ts:
        if not t.is_cuda or t.get_device() != dev:
            raise ValueError("all tensors must be on the same device")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")


def _fp8(t, name):
    if t.dtype not in (FP8, torch.uint8):
        raise TypeError(f"{name} must be float8_e4m3fn (or its uint8 bytes), got {t.dtype}")


def _f32(t, name):
    if t.dtype != torch.float32:
        raise TypeError(f"{name} must be float32, got {t.dtype}")


def _bf16(t, name):
    if t.dtype != torch.bfloat16:
        raise TypeError(f"{name} must be bfloat16, got {t.dtype}")


def _shape(t, shape, name):
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def version() -> int:
    return _lib.dg_version()


def select_config(kind: int, m: int, n: int, k: int, num_groups: int = 1, num_cus: int = 256) -> dict:
    """Tile configuration the heuristic picks (host only, no GPU needed)."""
    cfg = TileConfig()
    _check(_lib.dg_select_config(kind, m, n, k, num_groups, num_cus, ctypes.byref(cfg)),
           "dg_select_config")
    return {f: getattr(cfg, f) for f, _ in TileConfig._fields_}


# ---------------------------------------------------------------- C names ---

def dg_gemm_fp8_nt(a, sa, b, sb, c):
    """C[M,N] bf16 = fine-grained-scaled A[M,K] . B[N,K]^T (see include/dg.h)."""
    _fp8(a, "a"); _fp8(b, "b"); _f32(sa, "sa"); _f32(sb, "sb")
    m, k = a.shape
    n = b.shape[0]
    _shape(b, (n, k), "b"); _shape(sa, (m, k // 128), "sa"); _shape(sb, ((n + 127) // 128, k // 128), "sb")
    _shape(c, (m, n), "c")
    if c.dtype != torch.bfloat16:
        raise TypeError("c must be bfloat16")
    _dev(a, sa, b, sb, c)
    _check(_lib.dg_gemm_fp8_nt(_ptr(a), _ptr(sa), _ptr(b), _ptr(sb), _ptr(c), m, n, k, _stream(c)),
           "dg_gemm_fp8_nt")
    return c


def dg_gemm_fp8_nt_ue8m0(a, sa, b, sb, c):
    """dg_gemm_fp8_nt with power-of-two (UE8M0) scales applied by the
    block-scaled MFMA (see include/dg.h); sa, sb must be powers of two."""
    _fp8(a, "a"); _fp8(b, "b"); _f32(sa, "sa"); _f32(sb, "sb")
    m, k = a.shape
    n = b.shape[0]
    _shape(b, (n, k), "b"); _shape(sa, (m, k // 128), "sa"); _shape(sb, ((n + 127) // 128, k // 128), "sb")
    _shape(c, (m, n), "c")
    if c.dtype != torch.bfloat16:
        raise TypeError("c must be bfloat16")
    _dev(a, sa, b, sb, c)
    _check(_lib.dg_gemm_fp8_nt_ue8m0(_ptr(a), _ptr(sa), _ptr(b), _ptr(sb), _ptr(c), m, n, k, _stream(c)),
           "dg_gemm_fp8_nt_ue8m0")
    return c


def dg_gemm_fp8_nt_ue8m0_packed(a, sa, b, sb, c):
    """dg_gemm_fp8_nt_ue8m0 with packed UE8M0 scales: int32 words holding the
    biased exponents of four consecutive K blocks, block 4w+i in byte i
    (sa [M, ceil(K/512)], sb [ceil(N/128), ceil(K/512)]; see include/dg.h)."""
    _fp8(a, "a"); _fp8(b, "b")
    for t, name in ((sa, "sa"), (sb, "sb")):
        if t.dtype != torch.int32:
            raise TypeError(f"{name} must be int32 (packed UE8M0), got {t.dtype}")
    m, k = a.shape
    n = b.shape[0]
    kw = (k // 128 + 3) // 4
    _shape(b, (n, k), "b"); _shape(sa, (m, kw), "sa"); _shape(sb, ((n + 127) // 128, kw), "sb")
    _shape(c, (m, n), "c")
    if c.dtype != torch.bfloat16:
        raise TypeError("c must be bfloat16")
    _dev(a, sa, b, sb, c)
    _check(_lib.dg_gemm_fp8_nt_ue8m0_packed(_ptr(a), _ptr(sa), _ptr(b), _ptr(sb), _ptr(c), m, n, k, _stream(c)),
           "dg_gemm_fp8_nt_ue8m0_packed")
    return c


def dg_gemm_bf16_nt(a, b, c):
    """C[M,N] bf16 = A[M,K] bf16 . B[N,K]^T bf16, fp32 accumulation (see include/dg.h)."""
    for t, name in ((a, "a"), (b, "b"), (c, "c")):
        if t.dtype != torch.bfloat16:
            raise TypeError(f"{name} must be bfloat16, got {t.dtype}")
    m, k = a.shape
    n = b.shape[0]
    _shape(b, (n, k), "b"); _shape(c, (m, n), "c")
    _dev(a, b, c)
    _check(_lib.dg_gemm_bf16_nt(_ptr(a), _ptr(b), _ptr(c), m, n, k, _stream(c)), "dg_gemm_bf16_nt")
    return c


def _scale_cols(sa, sb, k, packed):
    """Columns of the scale tensors: K/128 fp32 scales, or ceil(K/512) int32
    words of packed UE8M0 exponents."""
    if not packed:
        _f32(sa, "sa"); _f32(sb, "sb")
        return k // 128
    for t, name in ((sa, "sa"), (sb, "sb")):
        if t.dtype != torch.int32:
            raise TypeError(f"{name} must be int32 (packed UE8M0), got {t.dtype}")
    return (k // 128 + 3) // 4


def dg_grouped_bf16_contiguous(a, b, c, m_indices):
    """Contiguous MoE layout in BF16: a [M_total,K], b [G,N,K], c [M_total,N]
    bf16, m_indices [M_total] int32 (see include/dg.h)."""
    for t, name in ((a, "a"), (b, "b"), (c, "c")):
        _bf16(t, name)
    m_total, k = a.shape
    g, n, _ = b.shape
    _shape(b, (g, n, k), "b"); _shape(c, (m_total, n), "c"); _shape(m_indices, (m_total,), "m_indices")
    if m_indices.dtype != torch.int32:
        raise TypeError("m_indices must be int32")
    _dev(a, b, c, m_indices)
    _check(_lib.dg_grouped_bf16_contiguous(_ptr(a), _ptr(b), _ptr(c), _ptr(m_indices), m_total, n, k, g, _stream(c)),
           "dg_grouped_bf16_contiguous")
    return c


def dg_grouped_bf16_masked(a, b, c, masked_m):
    """Masked MoE layout in BF16: a [G,M_max,K], b [G,N,K], c [G,M_max,N] bf16,
    masked_m [G] int32 (see include/dg.h)."""
    for t, name in ((a, "a"), (b, "b"), (c, "c")):
        _bf16(t, name)
    g, m_max, k = a.shape
    n = b.shape[1]
    _shape(b, (g, n, k), "b"); _shape(c, (g, m_max, n), "c"); _shape(masked_m, (g,), "masked_m")
    if masked_m.dtype != torch.int32:
        raise TypeError("masked_m must be int32")
    _dev(a, b, c, masked_m)
    _check(_lib.dg_grouped_bf16_masked(_ptr(a), _ptr(b), _ptr(c), _ptr(masked_m), g, m_max, n, k, _stream(c)),
           "dg_grouped_bf16_masked")
    return c


def dg_grouped_fp8_contiguous(a, sa, b, sb, c, m_indices):
    return _grouped_contiguous(_lib.dg_grouped_fp8_contiguous, "dg_grouped_fp8_contiguous", False,
                               a, sa, b, sb, c, m_indices)


def dg_grouped_fp8_contiguous_ue8m0_packed(a, sa, b, sb, c, m_indices):
    """dg_grouped_fp8_contiguous with packed UE8M0 scales (int32 words of four
    exponent bytes: sa [M_total, ceil(K/512)], sb [G, ceil(N/128), ceil(K/512)])."""
    return _grouped_contiguous(_lib.dg_grouped_fp8_contiguous_ue8m0_packed,
                               "dg_grouped_fp8_contiguous_ue8m0_packed", True, a, sa, b, sb, c, m_indices)


def _grouped_contiguous(fn, name, packed, a, sa, b, sb, c, m_indices):
    _fp8(a, "a"); _fp8(b, "b")
    m_total, k = a.shape
    g, n, _ = b.shape
    kc = _scale_cols(sa, sb, k, packed)
    _shape(b, (g, n, k), "b"); _shape(sa, (m_total, kc), "sa")
    _shape(sb, (g, (n + 127) // 128, kc), "sb"); _shape(c, (m_total, n), "c")
    _shape(m_indices, (m_total,), "m_indices")
    if m_indices.dtype != torch.int32:
        raise TypeError("m_indices must be int32")
    if c.dtype != torch.bfloat16:
        raise TypeError("c must be bfloat16")
    _dev(a, sa, b, sb, c, m_indices)
    _check(fn(_ptr(a), _ptr(sa), _ptr(b), _ptr(sb), _ptr(c), _ptr(m_indices), m_total, n, k, g, _stream(c)), name)
    return c


def dg_grouped_fp8_contiguous_swiglu(a, sa, b, sb, q, s, m_indices):
    """Contiguous grouped GEMM with B [G,2I,K] (gate rows | up rows), fused
    with SwiGLU and the 1x128 re-quantise: q fp8 [M_total,I], s fp32
    [M_total,I/128] (see include/dg.h)."""
    _fp8(a, "a"); _fp8(b, "b"); _f32(sa, "sa"); _f32(sb, "sb"); _fp8(q, "q"); _f32(s, "s")
    m_total, k = a.shape
    g, n, _ = b.shape
    if n % 256:
        raise ValueError(f"b must stack gate and up projections of a width that is a multiple of 128 (N={n})")
    i = n // 2
    _shape(b, (g, n, k), "b"); _shape(sa, (m_total, k // 128), "sa")
    _shape(sb, (g, n // 128, k // 128), "sb"); _shape(q, (m_total, i), "q"); _shape(s, (m_total, i // 128), "s")
    _shape(m_indices, (m_total,), "m_indices")
    if m_indices.dtype != torch.int32:
        raise TypeError("m_indices must be int32")
    _dev(a, sa, b, sb, q, s, m_indices)
    _check(_lib.dg_grouped_fp8_contiguous_swiglu(_ptr(a), _ptr(sa), _ptr(b), _ptr(sb), _ptr(q), _ptr(s),
                                                 _ptr(m_indices), m_total, n, k, g, _stream(q)),
           "dg_grouped_fp8_contiguous_swiglu")
    return q, s


def dg_grouped_fp8_masked(a, sa, b, sb, c, masked_m):
    return _grouped_masked(_lib.dg_grouped_fp8_masked, "dg_grouped_fp8_masked", a, sa, b, sb, c, masked_m)


def dg_grouped_fp8_masked_ue8m0_packed(a, sa, b, sb, c, masked_m):
    """dg_grouped_fp8_masked with packed UE8M0 scales (int32 words of four
    exponent bytes: sa [G, M_max, ceil(K/512)], sb [G, ceil(N/128), ceil(K/512)])."""
    return _grouped_masked(_lib.dg_grouped_fp8_masked_ue8m0_packed, "dg_grouped_fp8_masked_ue8m0_packed",
                           a, sa, b, sb, c, masked_m, packed=True)


def dg_grouped_fp8_masked_noalloc(a, sa, b, sb, c, masked_m):
    """dg_grouped_fp8_masked without any allocation (split-K partials in the
    library's fixed 64 MB scratch; usable under graph capture).  Calls that
    overlap on one GPU share the scratch and race."""
    return _grouped_masked(_lib.dg_grouped_fp8_masked_noalloc, "dg_grouped_fp8_masked_noalloc",
                           a, sa, b, sb, c, masked_m)


def _grouped_masked(fn, name, a, sa, b, sb, c, masked_m, packed=False):
    _fp8(a, "a"); _fp8(b, "b")
    g, m_max, k = a.shape
    n = b.shape[1]
    kc = _scale_cols(sa, sb, k, packed)
    _shape(b, (g, n, k), "b"); _shape(sa, (g, m_max, kc), "sa")
    _shape(sb, (g, (n + 127) // 128, kc), "sb"); _shape(c, (g, m_max, n), "c")
    _shape(masked_m, (g,), "masked_m")
    if masked_m.dtype != torch.int32:
        raise TypeError("masked_m must be int32")
    if c.dtype != torch.bfloat16:
        raise TypeError("c must be bfloat16")
    _dev(a, sa, b, sb, c, masked_m)
    _check(fn(_ptr(a), _ptr(sa), _ptr(b), _ptr(sb), _ptr(c), _ptr(masked_m), g, m_max, n, k, _stream(c)), name)
    return c


def dg_wgrad_fp8_nt(a, sa, b, sb, d):
    _fp8(a, "a"); _fp8(b, "b"); _f32(sa, "sa"); _f32(sb, "sb")
    m, k = a.shape
    n = b.shape[0]
    _shape(b, (n, k), "b"); _shape(sa, (m, k // 128), "sa"); _shape(sb, (n, k // 128), "sb")
    _shape(d, (m, n), "d"); _f32(d, "d")
    _dev(a, sa, b, sb, d)
    _check(_lib.dg_wgrad_fp8_nt(_ptr(a), _ptr(sa), _ptr(b), _ptr(sb), _ptr(d), m, n, k, _stream(d)),
           "dg_wgrad_fp8_nt")
    return d


def dg_k_grouped_wgrad_fp8_nt(a, sa, b, sb, d, ks):
    """ks: per-group token counts (host list/tuple of ints, multiples of 128)."""
    _fp8(a, "a"); _fp8(b, "b"); _f32(sa, "sa"); _f32(sb, "sb")
    ks = [int(x) for x in ks]
    g = len(ks)
    m, t = a.shape
    n = b.shape[0]
    if sum(ks) != t:
        raise ValueError(f"sum(ks)={sum(ks)} does not match the token dimension {t}")
    _shape(b, (n, t), "b"); _shape(sa, (m, t // 128), "sa"); _shape(sb, (n, t // 128), "sb")
    _shape(d, (g, m, n), "d"); _f32(d, "d")
    _dev(a, sa, b, sb, d)
    ks_arr = (ctypes.c_int32 * g)(*ks)
    _check(_lib.dg_k_grouped_wgrad_fp8_nt(_ptr(a), _ptr(sa), _ptr(b), _ptr(sb), _ptr(d), ks_arr, g, m, n,
                                          _stream(d)), "dg_k_grouped_wgrad_fp8_nt")
    return d


def dg_quantize_fp8_1x128(x, q, s):
    """x fp32 [M,K] -> q fp8 [M,K], s fp32 [M,K/128] (see include/dg.h)."""
    _f32(x, "x"); _fp8(q, "q"); _f32(s, "s")
    _dev(x, q, s)
    m, k = x.shape
    _shape(q, (m, k), "q"); _shape(s, (m, k // 128), "s")
    _check(_lib.dg_quantize_fp8_1x128(_ptr(x), _ptr(q), _ptr(s), m, k, _stream(x)), "dg_quantize_fp8_1x128")
    return q, s


def dg_quantize_fp8_128x128(x, q, s):
    """x fp32 [N,K] -> q fp8 [N,K], s fp32 [ceil(N/128),K/128] (see include/dg.h)."""
    _f32(x, "x"); _fp8(q, "q"); _f32(s, "s")
    _dev(x, q, s)
    n, k = x.shape
    _shape(q, (n, k), "q"); _shape(s, ((n + 127) // 128, k // 128), "s")
    _check(_lib.dg_quantize_fp8_128x128(_ptr(x), _ptr(q), _ptr(s), n, k, _stream(x)), "dg_quantize_fp8_128x128")
    return q, s


def _i32w(t, name):
    if t.dtype != torch.int32:
        raise TypeError(f"{name} must be int32 (packed UE8M0), got {t.dtype}")


def dg_quantize_fp8_1x128_ue8m0(x, q, s):
    """x fp32 [M,K] -> q fp8 [M,K], s int32 [M,ceil(K/512)]: power-of-two
    scales, packed UE8M0 (see include/dg.h)."""
    _f32(x, "x"); _fp8(q, "q"); _i32w(s, "s")
    _dev(x, q, s)
    m, k = x.shape
    _shape(q, (m, k), "q"); _shape(s, (m, (k // 128 + 3) // 4), "s")
    _check(_lib.dg_quantize_fp8_1x128_ue8m0(_ptr(x), _ptr(q), _ptr(s), m, k, _stream(x)),
           "dg_quantize_fp8_1x128_ue8m0")
    return q, s


def dg_quantize_fp8_128x128_ue8m0(x, q, s):
    """x fp32 [N,K] -> q fp8 [N,K], s int32 [ceil(N/128),ceil(K/512)]: power-of-two
    scales, packed UE8M0 (see include/dg.h)."""
    _f32(x, "x"); _fp8(q, "q"); _i32w(s, "s")
    _dev(x, q, s)
    n, k = x.shape
    _shape(q, (n, k), "q"); _shape(s, ((n + 127) // 128, (k // 128 + 3) // 4), "s")
    _check(_lib.dg_quantize_fp8_128x128_ue8m0(_ptr(x), _ptr(q), _ptr(s), n, k, _stream(x)),
           "dg_quantize_fp8_128x128_ue8m0")
    return q, s


def dg_quantize_fp8_1x128_transposed(x, q, s):
    """x fp32 [T,F] -> q fp8 [F,T], s fp32 [F,T/128] (see include/dg.h)."""
    _f32(x, "x"); _fp8(q, "q"); _f32(s, "s")
    _dev(x, q, s)
    t, f = x.shape
    _shape(q, (f, t), "q"); _shape(s, (f, t // 128), "s")
    _check(_lib.dg_quantize_fp8_1x128_transposed(_ptr(x), _ptr(q), _ptr(s), t, f, _stream(x)),
           "dg_quantize_fp8_1x128_transposed")
    return q, s


def _even_width(c):
    """(M, 2I) of the first GEMM's output c: the gate and up halves need an
    even width (an odd one would walk the rows with the wrong stride)."""
    if c.dim() != 2 or c.shape[1] % 2:
        raise ValueError(f"c must be [M, 2I] with an even width, got {tuple(c.shape)}")
    return c.shape


def dg_swiglu_quantize_fp8_1x128(c, q, s):
    """c bf16 [M,2I] (gate | up) -> q fp8 [M,I], s fp32 [M,I/128]: SwiGLU then
    the 1x128 quantise (see include/dg.h)."""
    _bf16(c, "c"); _fp8(q, "q"); _f32(s, "s")
    m, i2 = _even_width(c)
    _dev(c, q, s)
    i = i2 // 2
    _shape(q, (m, i), "q"); _shape(s, (m, i // 128), "s")
    _check(_lib.dg_swiglu_quantize_fp8_1x128(_ptr(c), _ptr(q), _ptr(s), m, i, _stream(c)),
           "dg_swiglu_quantize_fp8_1x128")
    return q, s


# ------------------------------------------------------ page-style names ---

def gemm_fp8_fp8_bf16_nt(lhs, rhs, out):
    return dg_gemm_fp8_nt(lhs[0], lhs[1], rhs[0], rhs[1], out)


def gemm_fp8_fp8_bf16_nt_ue8m0(lhs, rhs, out):
    """Power-of-two scales as fp32 values, or packed UE8M0 (int32 words)."""
    if lhs[1].dtype == torch.int32:
        return dg_gemm_fp8_nt_ue8m0_packed(lhs[0], lhs[1], rhs[0], rhs[1], out)
    return dg_gemm_fp8_nt_ue8m0(lhs[0], lhs[1], rhs[0], rhs[1], out)


def gemm_bf16_bf16_bf16_nt(lhs, rhs, out):
    return dg_gemm_bf16_nt(lhs, rhs, out)


def m_grouped_gemm_fp8_fp8_bf16_nt_contiguous(lhs, rhs, out, m_indices):
    """fp32 scales, or packed UE8M0 (int32 words)."""
    if lhs[1].dtype == torch.int32:
        return dg_grouped_fp8_contiguous_ue8m0_packed(lhs[0], lhs[1], rhs[0], rhs[1], out, m_indices)
    return dg_grouped_fp8_contiguous(lhs[0], lhs[1], rhs[0], rhs[1], out, m_indices)


def m_grouped_gemm_fp8_fp8_fp8_nt_contiguous_swiglu(lhs, rhs, m_indices):
    """First expert linear layer + SwiGLU + 1x128 re-quantise: returns the
    second layer's operand (fp8 [M_total,I], fp32 scales [M_total,I/128]);
    rows of padding (-1) are left as torch.empty gives them."""
    m_total = lhs[0].shape[0]
    i = rhs[0].shape[1] // 2
    dev = lhs[0].device
    return dg_grouped_fp8_contiguous_swiglu(
        lhs[0], lhs[1], rhs[0], rhs[1], torch.empty((m_total, i), dtype=FP8, device=dev),
        torch.empty((m_total, i // 128), dtype=torch.float32, device=dev), m_indices)


def m_grouped_gemm_bf16_bf16_bf16_nt_contiguous(lhs, rhs, out, m_indices):
    return dg_grouped_bf16_contiguous(lhs, rhs, out, m_indices)


def m_grouped_gemm_bf16_bf16_bf16_nt_masked(lhs, rhs, out, masked_m):
    return dg_grouped_bf16_masked(lhs, rhs, out, masked_m)


def m_grouped_gemm_fp8_fp8_bf16_nt_masked(lhs, rhs, out, masked_m):
    """fp32 scales, or packed UE8M0 (int32 words)."""
    if lhs[1].dtype == torch.int32:
        return dg_grouped_fp8_masked_ue8m0_packed(lhs[0], lhs[1], rhs[0], rhs[1], out, masked_m)
    return dg_grouped_fp8_masked(lhs[0], lhs[1], rhs[0], rhs[1], out, masked_m)


def wgrad_gemm_fp8_fp8_fp32_nt(lhs, rhs, out):
    return dg_wgrad_fp8_nt(lhs[0], lhs[1], rhs[0], rhs[1], out)


def k_grouped_wgrad_gemm_fp8_fp8_fp32_nt(lhs, rhs, out, ks):
    return dg_k_grouped_wgrad_fp8_nt(lhs[0], lhs[1], rhs[0], rhs[1], out, ks)


def quantize_fp8_1x128(x):
    """Activations: (fp8 [M,K], fp32 scales [M,K/128]) for the GEMM calls above."""
    m, k = x.shape
    return dg_quantize_fp8_1x128(x, torch.empty((m, k), dtype=FP8, device=x.device),
                                 torch.empty((m, k // 128), dtype=torch.float32, device=x.device))


def quantize_fp8_128x128(x):
    """Weights: (fp8 [N,K], fp32 scales [ceil(N/128),K/128])."""
    n, k = x.shape
    return dg_quantize_fp8_128x128(x, torch.empty((n, k), dtype=FP8, device=x.device),
                                   torch.empty(((n + 127) // 128, k // 128), dtype=torch.float32, device=x.device))


def quantize_fp8_1x128_ue8m0(x):
    """Activations with power-of-two scales: (fp8 [M,K], packed UE8M0 int32 [M,ceil(K/512)])."""
    m, k = x.shape
    return dg_quantize_fp8_1x128_ue8m0(x, torch.empty((m, k), dtype=FP8, device=x.device),
                                       torch.empty((m, (k // 128 + 3) // 4), dtype=torch.int32, device=x.device))


def quantize_fp8_128x128_ue8m0(x):
    """Weights with power-of-two scales: (fp8 [N,K], packed UE8M0 int32 [ceil(N/128),ceil(K/512)])."""
    n, k = x.shape
    return dg_quantize_fp8_128x128_ue8m0(x, torch.empty((n, k), dtype=FP8, device=x.device),
                                         torch.empty(((n + 127) // 128, (k // 128 + 3) // 4), dtype=torch.int32,
                                                     device=x.device))


def quantize_fp8_1x128_transposed(x):
    """Weight-gradient operand from x [T,F]: (fp8 [F,T], fp32 scales [F,T/128])."""
    t, f = x.shape
    return dg_quantize_fp8_1x128_transposed(x, torch.empty((f, t), dtype=FP8, device=x.device),
                                            torch.empty((f, t // 128), dtype=torch.float32, device=x.device))


def swiglu_quantize_fp8_1x128(c):
    """Second-GEMM operand from the first GEMM's bf16 output c [M,2I]:
    (fp8 silu(gate)*up [M,I], fp32 scales [M,I/128])."""
    m, i2 = _even_width(c)
    i = i2 // 2
    return dg_swiglu_quantize_fp8_1x128(c, torch.empty((m, i), dtype=FP8, device=c.device),
                                        torch.empty((m, i // 128), dtype=torch.float32, device=c.device))
