"""Parity bounds of the FP8 (E4M3) forward, derived from its arithmetic.

Q, K and V reach the kernel and the oracle as the same E4M3 codes (times
their float32 descales).  Products of E4M3 values are exact in float32 and
the scores, exponentials and sums run in float32, so the one coarse rounding
is that of the probabilities to E4M3 before the second product.

How that rounding enters.  For row i and key j the kernel rounds
x_ij = 2^(c s_ij - m_t + 6), where m_t is the row's running maximum (log2
units) when key j's tile is processed.  The running maximum trails the true
one by at most 2, so x_ij lies in (0, 2^8], inside the format's range.  The
row sum adds the unrounded x_ij, so the weight of key j in the output is
P_ij = x_ij 2^(m_t - m_f) / l_i with the final maximum m_f and
l_i = sum_j x_ij 2^(m_t - m_f) >= 2^6 (the key with the largest score
contributes at least 2^6).  Rounding to nearest even in E4M3:
  * x >= 2^-6 (normal binades, 3 mantissa bits): |dx| <= 2^-4 x,
    so |dP_ij| <= 2^-4 P_ij;
  * x <  2^-6 (subnormals, spacing 2^-9): |dx| <= 2^-10, so
    |dP_ij| <= 2^-10 / l_i <= 2^-16, while P_ij <= x / l_i < 2^-12.
Hence every visible key obeys |dP_ij| <= e_ij := 2^-4 max(P_ij, 2^-12).

Worst case (every rounding against the same sign), per element:
  |dO_ic| <= (1 + 2^-8) (sum_j e_ij |V_jc| + 2^-10 sum_j P_ij |V_jc|)
             + 2^-8 |O_ic|
where 2^-8 |O| is the bfloat16 output rounding and the 2^-10 term covers the
float32 arithmetic (score sums over d, exp2, the row and product sums; each
below (d + Nk) 2^-24 relative at these sizes).

Statistical bound.  A rounding to nearest has an error uniform over half a
spacing around the exact value, so its variance is at most (bound)^2 / 3 for
both the E4M3 and the bfloat16 rounding; with independent roundings
  sigma_ic^2 = (1/3) sum_j e_ij^2 V_jc^2 + (1/3) (2^-8 O_ic)^2
bounds the variance of dO_ic, and the root mean square of dO_ic / sigma_ic
over all elements is at most 1 in expectation.  That is the check; unlike a
bound in units of V, it scales with each row's own output, so an output
scaled by 1.1, halved on some rows, or missing one key tile fails it
(tests/test_fp8_check.py plants each of these in the oracle's own output).

LSE comes from float32 row sums of the unrounded values: max abs error
<= 1e-3, as for the 16-bit path.

This module checks a result against the float64 oracle's own P; it runs on
the CPU and is used by the GPU FP8 parity tests.
"""

from __future__ import annotations

import math

import numpy as np

from oracle import attention_f64 as orc

E4M3_REL = 2.0 ** -4      # half spacing of a 3-bit mantissa, relative
P_FLOOR = 2.0 ** -12      # weights below this may come from subnormal x
BF16_REL = 2.0 ** -8      # bfloat16 output rounding, relative
F32_SLACK = 2.0 ** -10    # float32 arithmetic, relative to sum_j P |V|
RMS_LIMIT = 1.0           # expected-value bound of rms(dO / sigma)
LSE_TOL = 1e-3


def decoded(codes, descale: float) -> np.ndarray:
    """float64 values of E4M3 codes (uint8 array) times their descale."""
    return orc.fp8_e4m3_decode(np.asarray(codes, dtype=np.uint8)) * descale


def check_fp8_output(o, lse, q, k, v, scale: float, causal: bool, row_ids=None, nq_total=None):
    """Check an FP8 forward's O [B, Hq, Nq, d] and LSE [B, Hq, Nq] (float64
    arrays) against the float64 oracle on the decoded inputs q, k, v.
    ``row_ids``/``nq_total`` select rows of a longer query sequence (q, o and
    lse then hold only those rows).  Raises AssertionError on a violation;
    returns the statistics."""
    o = np.asarray(o, dtype=np.float64)
    lse = np.asarray(lse, dtype=np.float64)
    bsz, hq, nq, d = q.shape
    g = hq // k.shape[1]
    worst_ratio, sq_sum, count, lse_err = 0.0, 0.0, 0, 0.0
    for b in range(bsz):
        for h in range(hq):
            kh, vh = k[b, h // g], v[b, h // g]
            p, rl = orc.attention_probs(q[b, h], kh, scale, causal, row_ids, nq_total)
            ro = p @ vh
            vis = orc.visible_mask(nq, kh.shape[0], causal, row_ids, nq_total)
            e = np.where(vis, E4M3_REL * np.maximum(p, P_FLOOR), 0.0)
            absv = np.abs(vh)
            worst = (1 + BF16_REL) * (e @ absv + F32_SLACK * (p @ absv)) + BF16_REL * np.abs(ro)
            sigma = np.sqrt(((e * e) @ (vh * vh) + (BF16_REL * ro) ** 2) / 3.0)
            got, gl = o[b, h], lse[b, h]
            assert not np.isnan(got).any(), f"O[{b},{h}]: NaN"
            empty = np.isneginf(rl)
            assert np.array_equal(np.isneginf(gl), empty), f"LSE[{b},{h}]: rows without keys differ"
            assert (got[empty] == 0).all(), f"O[{b},{h}]: rows without keys must be 0"
            err = np.abs(got - ro)
            ratio = err / np.maximum(worst, 1e-300)
            i, c = np.unravel_index(np.argmax(ratio), ratio.shape)
            assert ratio[i, c] <= 1.0, (f"O[{b},{h}] row {i} col {c}: |dO| {err[i, c]:.4e} above the worst-case "
                                        f"bound {worst[i, c]:.4e}")
            live = sigma > 0
            assert (err[~live] == 0).all(), f"O[{b},{h}]: error where no rounding can reach"
            sq_sum += float(np.sum((err[live] / sigma[live]) ** 2))
            count += int(live.sum())
            worst_ratio = max(worst_ratio, float(ratio[i, c]))
            if (~empty).any():
                lse_err = max(lse_err, float(np.abs(gl[~empty] - rl[~empty]).max()))
    rms = math.sqrt(sq_sum / max(count, 1))
    assert rms <= RMS_LIMIT, f"rms(dO / sigma) = {rms:.3f} above {RMS_LIMIT} (expected-value bound)"
    assert lse_err <= LSE_TOL, f"LSE max abs error {lse_err:.4e} > {LSE_TOL}"
    return {"rms_over_sigma": rms, "worst_over_bound": worst_ratio, "lse_err": lse_err}
