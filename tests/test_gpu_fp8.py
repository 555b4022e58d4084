"""GPU parity of the FP8 (E4M3) forward against the float64 oracle on the
decoded inputs.

Tolerance (derived from the arithmetic).  Q, K and V reach the kernel and the
oracle as the same E4M3 codes, products of E4M3 values are exact in float32,
and the scores are accumulated in float32, so the one coarse rounding is that
of the probabilities to E4M3 before the second product (relative error at
most 2^-4; the row sum keeps the unrounded float32 values).  For row i,
|dO_i| <= 2^-4 * max|V| in the worst case (every probability rounded the same
way), and with independent rounding directions the root-mean-square error is
at most 2^-4/sqrt(3) * rms(V).  Both are checked, with 2^-8 * max|V| added to
the first for the bf16 output rounding.  LSE comes from float32 row sums of
the unrounded values: max abs error <= 1e-3, as for the 16-bit path.
"""

from __future__ import annotations

import math

import numpy as np
import pytest
import torch

from parity import dev, f64
from oracle import attention_f64 as orc
import synth_inputs as si

pytestmark = pytest.mark.gpu


def _codes(t: torch.Tensor) -> np.ndarray:
    return t.view(torch.uint8).numpy()


def check_fp8(q, k, v, desc, causal, scale=None, rows=None):
    import exact_io_aware_47_amd as fa
    d = q.shape[-1]
    sc = 1.0 / math.sqrt(d) if scale is None else scale
    o, lse = fa.fwd_fp8(dev(q), dev(k), dev(v), *desc, causal=causal, scale=scale)
    torch.cuda.synchronize()
    o, lse = f64(o.cpu()), f64(lse.cpu())
    ro, rl = orc.attention_fwd_fp8(_codes(q), _codes(k), _codes(v), *desc, sc, causal)
    vmax = np.abs(orc.fp8_e4m3_decode(_codes(v)) * desc[2]).max()
    vrms = math.sqrt(np.mean((orc.fp8_e4m3_decode(_codes(v)) * desc[2]) ** 2))
    assert np.array_equal(np.isinf(lse), np.isinf(rl)), "rows without keys differ"
    fin = np.isfinite(rl)
    err = np.abs(o - ro)
    assert not np.isnan(o).any()
    max_tol = (2.0 ** -4 + 2.0 ** -8) * vmax
    rms = math.sqrt(np.mean(err ** 2))
    assert err.max() <= max_tol, f"O max abs error {err.max():.4e} > {max_tol:.4e}"
    assert rms <= 2.0 ** -4 / math.sqrt(3) * vrms, f"O rms error {rms:.4e} > {2.0 ** -4 / math.sqrt(3) * vrms:.4e}"
    lerr = np.abs(lse[fin] - rl[fin]).max() if fin.any() else 0.0
    assert lerr <= 1e-3, f"LSE max abs error {lerr:.4e}"
    return err.max(), rms, lerr


# B, Hq, Hkv, Nq, Nk, d, causal
CASES = [
    (1, 2, 2, 200, 200, 128, True),
    (2, 4, 2, 129, 300, 64, False),
    (1, 2, 1, 77, 77, 64, True),
    (1, 4, 4, 1000, 1000, 128, False),
    (1, 2, 2, 300, 100, 128, True),    # more queries than keys: rows without keys
    (1, 2, 2, 64, 1000, 128, True),
    (1, 1, 1, 1, 1, 64, False),
    (2, 8, 2, 513, 513, 128, True),
]


@pytest.mark.parametrize("B,Hq,Hkv,Nq,Nk,d,causal", CASES,
                         ids=[f"B{c[0]}_H{c[1]}x{c[2]}_N{c[3]}x{c[4]}_d{c[5]}_{'c' if c[6] else 'nc'}" for c in CASES])
def test_fp8_matches_oracle(B, Hq, Hkv, Nq, Nk, d, causal):
    print(f"fp8 case B={B} H={Hq}x{Hkv} N={Nq}x{Nk} d={d} causal={causal}", flush=True)
    q, k, v, desc = si.make_fp8_inputs(B, Hq, Hkv, Nq, Nk, d, seed=7000 + Nq + 3 * Nk + d)
    check_fp8(q, k, v, desc, causal)


@pytest.mark.parametrize("scale", [0.0, -0.2])
def test_fp8_unusual_scale(scale):
    q, k, v, desc = si.make_fp8_inputs(1, 2, 2, 150, 150, 128, seed=71)
    for causal in (False, True):
        check_fp8(q, k, v, desc, causal, scale=scale)


def test_fp8_unit_descales():
    """Codes used directly (descale 1): values up to the format's largest."""
    gen = torch.Generator().manual_seed(72)
    q, k, v = (torch.randn(1, 2, 160, 64, generator=gen).to(torch.float8_e4m3fn) for _ in range(3))
    check_fp8(q, k, v, (1.0, 1.0, 1.0), True)


def test_fp8_workload_mha_fp8_4k():
    w = si.WORKLOADS["mha_fp8_4k"]
    q, k, v, desc = si.make_fp8_inputs(w.B, w.Hq, w.Hkv, w.Nq, w.Nk, w.d, w.seed)
    import exact_io_aware_47_amd as fa
    o, lse = fa.fwd_fp8(dev(q), dev(k), dev(v), *desc, causal=True)
    torch.cuda.synchronize()
    o, lse = o.cpu(), lse.cpu()
    for b, h in ((0, 0), (1, 11)):
        sl = (slice(b, b + 1), slice(h, h + 1))
        ro, rl = orc.attention_fwd_fp8(_codes(q[sl]), _codes(k[sl]), _codes(v[sl]), *desc, w.scale, True)
        vd = orc.fp8_e4m3_decode(_codes(v[sl])) * desc[2]
        err = np.abs(f64(o[sl]) - ro)
        assert err.max() <= (2.0 ** -4 + 2.0 ** -8) * np.abs(vd).max(), f"O[{b},{h}] max abs error {err.max():.4e}"
        assert math.sqrt(np.mean(err ** 2)) <= 2.0 ** -4 / math.sqrt(3) * math.sqrt(np.mean(vd ** 2))
        assert np.abs(f64(lse[sl]) - rl).max() <= 1e-3
