"""Shared helpers of the GPU parity tests: device transfer, oracle calls on the
exact values the kernels see, and the tolerances.

Tolerances (written once, here):
* float32 path: normwise relative error max|x - ref| / max|ref| <= 1e-5 for
  O, LSE and every gradient (the tutorial's numerical-validation section asks
  the forward to agree with a float64 reference to about 1e-5 relative).
* float16 / bfloat16 with N(0,1) inputs: max abs error <= 2e-2 on O and
  <= 5e-2 on dQ, dK, dV; LSE (float32 output, scores accumulated in float32)
  max abs error <= 1e-3.
* float16 / bfloat16 with large logits (Q, K scaled up): gradients can reach
  tens, where the storage rounding of a 16-bit output alone exceeds 5e-2, so
  they are held to max|x - ref| / max(1, max|ref|) <= 5e-2.
Rows that see no key must give LSE = -inf on both sides (and O = 0).
"""

from __future__ import annotations

import math
import os
import sys

import numpy as np
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

TOL_F32_NORMWISE = 1e-5
TOL_O_16 = 2e-2
TOL_GRAD_16 = 5e-2
TOL_LSE_16 = 1e-3


def dev(t: torch.Tensor) -> torch.Tensor:
    return t.to("cuda").contiguous()


def f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu", torch.float64).numpy()


def _finite_split(got: np.ndarray, ref: np.ndarray, what: str):
    gi, ri = np.isinf(got), np.isinf(ref)
    assert np.array_equal(gi, ri), f"{what}: infinite entries differ ({gi.sum()} vs {ri.sum()})"
    if gi.any():
        assert np.array_equal(got[gi], ref[ri]), f"{what}: signs of infinite entries differ"
    assert not np.isnan(got).any(), f"{what}: NaN in result"
    return got[~gi], ref[~ri]


def err_stats(got: np.ndarray, ref: np.ndarray):
    if ref.size == 0:
        return 0.0, 0.0
    diff = np.abs(got - ref)
    return float(diff.max()), float(np.abs(ref).max())


def assert_close(what: str, got, ref, dtype: str, kind: str, large_logits: bool = False):
    """kind: 'o', 'lse' or 'grad'."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, f"{what}: shape {got.shape} vs {ref.shape}"
    g, r = _finite_split(got, ref, what)
    max_err, max_ref = err_stats(g, r)
    if dtype == "f32":
        rel = max_err / max(max_ref, 1e-30)
        assert rel <= TOL_F32_NORMWISE, f"{what}: normwise relative error {rel:.3e} > {TOL_F32_NORMWISE}"
        return rel
    if kind == "o":
        assert max_err <= TOL_O_16, f"{what}: max abs error {max_err:.4e} > {TOL_O_16}"
    elif kind == "lse":
        assert max_err <= TOL_LSE_16, f"{what}: max abs error {max_err:.4e} > {TOL_LSE_16}"
    elif kind == "grad":
        if large_logits:
            rel = max_err / max(1.0, max_ref)
            assert rel <= TOL_GRAD_16, f"{what}: scaled error {rel:.4e} > {TOL_GRAD_16} (raw {max_err:.3e})"
        else:
            assert max_err <= TOL_GRAD_16, f"{what}: max abs error {max_err:.4e} > {TOL_GRAD_16}"
    else:
        raise ValueError(kind)
    return max_err


def dtype_name(t: torch.Tensor) -> str:
    return {torch.float32: "f32", torch.float16: "f16", torch.bfloat16: "bf16"}[t.dtype]


def scale_for(d: int) -> float:
    return 1.0 / math.sqrt(d)
