"""Shared helpers for the tests (no method arithmetic here: conversions and
comparisons only)."""
import hashlib

import numpy as np
import torch

import oracle as O
from synthetic import bf16_bits_numpy, f32_numpy

# Tolerance for fp32 outputs against the fp64 oracle.
FROB_TOL = 1e-3
ELEM_TOL = 4e-3


def assert_close(got, ref, what=""):
    """relative Frobenius <= 1e-3 and max |err|/(|ref|+1) <= 4e-3."""
    fro = O.relative_frobenius(got, ref)
    el = O.elementwise_ratio(got, ref)
    assert fro <= FROB_TOL and el <= ELEM_TOL, f"{what}: rel-Frobenius {fro:.3e}, elementwise {el:.3e}"
    return fro, el


def bits(t: torch.Tensor):
    return bf16_bits_numpy(t)


def f32(t: torch.Tensor):
    return f32_numpy(t)


def same_bits(a: torch.Tensor, b: torch.Tensor) -> bool:
    """memcmp of two tensors' storage bytes (NaN-safe, -0 != +0)."""
    a = a.detach().contiguous().cpu().reshape(-1)
    b = b.detach().contiguous().cpu().reshape(-1)
    if a.shape != b.shape or a.dtype != b.dtype:
        return False
    return a.view(torch.uint8).numpy().tobytes() == b.view(torch.uint8).numpy().tobytes()


def digest(t: torch.Tensor) -> str:
    return hashlib.sha256(t.detach().contiguous().cpu().reshape(-1).view(torch.uint8).numpy().tobytes()).hexdigest()


def rne_bf16(t: torch.Tensor) -> torch.Tensor:
    """torch's CPU fp32 -> bf16 conversion (round to nearest, ties to even)."""
    return t.detach().cpu().to(torch.bfloat16)


def count_rows_differing(ref_row: torch.Tensor, rows: list) -> int:
    return sum(0 if same_bits(ref_row, r) else 1 for r in rows)


def d_major(v):
    """Value pages [P, Hkv, page, D] (token-major, as tests write them) in the
    d-major layout the library and the oracle take: [P, Hkv, D, page]."""
    if isinstance(v, torch.Tensor):
        return v.transpose(2, 3).contiguous()
    return np.ascontiguousarray(np.swapaxes(v, 2, 3))
