"""GPU parity of the FP8 (E4M3) forward against the float64 oracle on the
decoded inputs.

The tolerance is derived from the arithmetic in tests/fp8_check.py: per
element, the probabilities' rounding to E4M3 perturbs the weight of key j by
at most 2^-4 max(P_ij, 2^-12), which gives a worst-case bound on every
output element and a standard deviation sigma_ic from which the root mean
square of dO / sigma must stay at most 1; both scale with each row's own
output.  LSE: max abs error <= 1e-3.
"""

from __future__ import annotations

import math

import numpy as np
import pytest
import torch

from fp8_check import check_fp8_output, decoded
from parity import dev, f64
import synth_inputs as si

pytestmark = pytest.mark.gpu


def _codes(t: torch.Tensor) -> np.ndarray:
    return t.view(torch.uint8).numpy()


def _decoded(q, k, v, desc):
    return decoded(_codes(q), desc[0]), decoded(_codes(k), desc[1]), decoded(_codes(v), desc[2])


def check_fp8(q, k, v, desc, causal, scale=None):
    import exact_io_aware_47_amd as fa
    d = q.shape[-1]
    sc = 1.0 / math.sqrt(d) if scale is None else scale
    o, lse = fa.fwd_fp8(dev(q), dev(k), dev(v), *desc, causal=causal, scale=scale)
    torch.cuda.synchronize()
    qd, kd, vd = _decoded(q, k, v, desc)
    return check_fp8_output(f64(o.cpu()), f64(lse.cpu()), qd, kd, vd, sc, causal)


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
    """The benchmarked launch, compared on eight whole heads of both batches."""
    w = si.WORKLOADS["mha_fp8_4k"]
    q, k, v, desc = si.make_fp8_inputs(w.B, w.Hq, w.Hkv, w.Nq, w.Nk, w.d, w.seed)
    import exact_io_aware_47_amd as fa
    o, lse = fa.fwd_fp8(dev(q), dev(k), dev(v), *desc, causal=True)
    torch.cuda.synchronize()
    o, lse = o.cpu(), lse.cpu()
    for b, h in ((0, 0), (0, 5), (0, 9), (0, 15), (1, 0), (1, 7), (1, 11), (1, 15)):
        sl = (slice(b, b + 1), slice(h, h + 1))
        qd, kd, vd = _decoded(q[sl], k[sl], v[sl], desc)
        st = check_fp8_output(f64(o[sl]), f64(lse[sl]), qd, kd, vd, w.scale, True)
        print(f"fp8 4k head ({b},{h}): {st}", flush=True)
