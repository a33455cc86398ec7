"""Helpers for the GPU parity tests: device upload, sentinel outputs and the
parity bar against the oracle.

The bar (per call, over the outputs the call must write):
    |gpu - ref| <= 2^-7 * |ref| + 1e-3 * max|ref|   for every element, and
    ||gpu - ref||_F <= 2e-3 * ||ref||_F,
where ref is the oracle's rounded result (bf16, or fp32 for weight
gradients).  2^-7 is one bf16 unit in the last place relative to the value:
the GPU accumulates in fp32 in another order, so its bf16 may land one step
from the oracle's; the 1e-3*max term absorbs cancellation near zero.
Outputs the call must not write keep their sentinel bits exactly.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

SENTINEL_BF16 = 0xFFFF  # a NaN pattern the kernels never produce
ELEM_REL = 2.0 ** -7
ELEM_ABS = 1e-3
FRO_REL = 2e-3


def say(msg: str):
    """Name the case before a GPU step, flushed, so a failing run shows it."""
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def dev(x: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x)).to("cuda")


def sentinel_bf16(shape) -> torch.Tensor:
    return torch.full(shape, -1, dtype=torch.int16, device="cuda").view(torch.bfloat16)


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def bits_to_f64(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def check_close(got, ref, what: str):
    got = np.asarray(got, np.float64).ravel()
    ref = np.asarray(ref, np.float64).ravel()
    assert got.size == ref.size and ref.size > 0, what
    assert np.all(np.isfinite(got)), f"{what}: non-finite GPU values"
    mx = np.abs(ref).max()
    bound = ELEM_REL * np.abs(ref) + ELEM_ABS * mx
    err = np.abs(got - ref)
    bad = np.flatnonzero(err > bound)
    if bad.size:
        i = bad[np.argmax(err[bad] / bound[bad])]
        raise AssertionError(f"{what}: {bad.size}/{ref.size} elements outside the bound; worst flat index "
                             f"{i}: gpu={got[i]!r} ref={ref[i]!r} bound={bound[i]:.3g}")
    fro = np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300)
    assert fro <= FRO_REL, f"{what}: relative Frobenius error {fro:.3g} > {FRO_REL}"
    return float(err.max() / max(mx, 1e-300)), float(fro)
