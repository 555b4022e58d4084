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
* O of the large-logit workload (Q, K scaled by 8): its rows are nearly
  one-hot, so O is close to single rows of V and the two bfloat16 roundings
  the method makes (P before the second product, O at the end, each at most
  2^-8 relative) reach 2 * 2^-8 * max|V|, about 0.04, beyond the N(0,1)
  clause's 2e-2.  It is held instead to a bound derived per element from the
  oracle's own P (``assert_o_within_rounding``): the worst case
      |dO_ic| <= (1 + 2^-8) sum_j (2^-8 + 2 eps_i + g) P_ij |V_jc| + 2^-8 |O_ic|
  with eps_i the float32 error bound of row i's scores (natural-log units,
  d * 2^-24 * c * sum_d |q_id k_jd|, times 2 for the normalisation) and
  g = Nk * 2^-24 for the float32 sums over keys; and, since each rounding is
  uniform over half a spacing, rms(dO / sigma) <= 1 with
  sigma_ic^2 = (2^-8)^2 (sum_j P_ij^2 V_jc^2 + O_ic^2) / 3.
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


BF16_U = 2.0 ** -8   # unit roundoff of a 16-bit float with an 8-bit significand (bfloat16)
F32_U = 2.0 ** -24


def assert_o_within_rounding(what: str, got, q, k, v, scale: float, causal: bool, row_ids=None, nq_total=None):
    """O of one (batch, head) within the per-element rounding bound described
    in the module docstring.  q [nq, d] (the selected rows), k, v [nk, d], all
    float64 holding the exact 16-bit inputs; got [nq, d].  Returns
    (max abs error, rms of dO / sigma, max of dO / worst-case bound)."""
    from oracle import attention_f64 as orc
    got = np.asarray(got, dtype=np.float64)
    p, lse = orc.attention_probs(q, k, scale, causal, row_ids, nq_total)
    ref = p @ v
    nk, d = k.shape
    vis = orc.visible_mask(q.shape[0], nk, causal, row_ids, nq_total)
    # Float32 score error of each row in natural-log units (worst case over its keys).
    s_abs = abs(scale) * (np.abs(q) @ np.abs(k).T)
    gamma_d = d * F32_U / (1 - d * F32_U)
    eps = gamma_d * np.where(vis, s_abs, 0.0).max(axis=1) + 4 * F32_U
    rel = BF16_U + 2 * eps[:, None] + nk * F32_U
    worst = (1 + BF16_U) * ((rel * p) @ np.abs(v)) + BF16_U * np.abs(ref)
    sigma = BF16_U * np.sqrt(((p * p) @ (v * v) + ref * ref) / 3.0)
    assert not np.isnan(got).any(), f"{what}: NaN"
    empty = np.isneginf(lse)
    assert (got[empty] == 0).all(), f"{what}: rows without keys must be 0"
    err = np.abs(got - ref)
    ratio = err / np.maximum(worst, 1e-300)
    i, c = np.unravel_index(np.argmax(ratio), ratio.shape)
    assert ratio[i, c] <= 1.0, f"{what}: row {i} col {c} |dO| {err[i, c]:.4e} above its bound {worst[i, c]:.4e}"
    live = sigma > 0
    assert (err[~live] == 0).all(), f"{what}: error where no rounding can reach"
    rms = float(np.sqrt(np.mean((err[live] / sigma[live]) ** 2))) if live.any() else 0.0
    assert rms <= 1.0, f"{what}: rms(dO / sigma) = {rms:.3f} above 1"
    return float(err.max()), rms, float(ratio[i, c])
