"""CPU tests of the FP8 parity check (tests/fp8_check.py): it accepts an
output carrying exactly the rounding the FP8 forward performs, and rejects
outputs with planted mistakes of the kind a product or staging error makes.

The accepted output is built here from the oracle's scores: each row's
x = 2^6 exp(s - max) is rounded to E4M3 by torch's float8_e4m3fn cast (round
to nearest even), O = sum_j x_j V_j / sum_j x_j (the unrounded sum), and O is
rounded to bfloat16.  The mistakes are planted in that output.
"""

from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import synth_inputs as si
from fp8_check import check_fp8_output, decoded
from oracle import attention_f64 as orc

N = 640        # several 64-key tiles and rows well past 256
D = 128


def _inputs(causal: bool):
    q, k, v, desc = si.make_fp8_inputs(1, 2, 1, N, N, D, seed=4711 + causal)
    qd = decoded(q.view(torch.uint8).numpy(), desc[0])
    kd = decoded(k.view(torch.uint8).numpy(), desc[1])
    vd = decoded(v.view(torch.uint8).numpy(), desc[2])
    return qd, kd, vd


def _rounded_like_the_kernel(q, k, v, scale, causal, drop_keys=None, drop_from_row=0):
    """O and LSE with the FP8 forward's one coarse rounding (P to E4M3).
    drop_keys: a key range whose products are left out (a planted mistake)
    for rows >= drop_from_row; the row sum still counts those keys."""
    bsz, hq, nq, d = q.shape
    g = hq // k.shape[1]
    o = np.zeros((bsz, hq, nq, d))
    lse = np.zeros((bsz, hq, nq))
    for b in range(bsz):
        for h in range(hq):
            s = scale * (q[b, h] @ k[b, h // g].T)
            vis = orc.visible_mask(nq, s.shape[1], causal)
            s = np.where(vis, s, -np.inf)
            mx = s.max(axis=1, keepdims=True)
            x = np.where(vis, 2.0 ** 6 * np.exp(s - mx), 0.0)
            xr = torch.from_numpy(x).float().to(torch.float8_e4m3fn).double().numpy()
            if drop_keys is not None:
                xr[drop_from_row:, drop_keys] = 0.0
            l = x.sum(axis=1, keepdims=True)
            o[b, h] = (xr @ v[b, h // g]) / l
            lse[b, h] = (mx + np.log(l) - 6 * math.log(2.0))[:, 0]
    o = torch.from_numpy(o).to(torch.bfloat16).double().numpy()
    return o, lse


@pytest.mark.parametrize("causal", [True, False])
def test_check_accepts_e4m3_rounded_output(causal):
    q, k, v = _inputs(causal)
    sc = 1.0 / math.sqrt(D)
    o, lse = _rounded_like_the_kernel(q, k, v, sc, causal)
    stats = check_fp8_output(o, lse, q, k, v, sc, causal)
    # The bound holds in expectation; the real rounding sits well inside it.
    assert stats["rms_over_sigma"] < 0.9 and stats["worst_over_bound"] < 1.0


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("mistake", ["halved past row 256", "scaled by 1.1", "one key tile missing",
                                     "scaled by 1.03"])
def test_check_rejects_planted_mistake(causal, mistake):
    q, k, v = _inputs(causal)
    sc = 1.0 / math.sqrt(D)
    if mistake == "one key tile missing":
        o, lse = _rounded_like_the_kernel(q, k, v, sc, causal, drop_keys=slice(64, 128), drop_from_row=256)
    else:
        o, lse = _rounded_like_the_kernel(q, k, v, sc, causal)
        if mistake == "halved past row 256":
            o[:, :, 256:] *= 0.5
        elif mistake == "scaled by 1.1":
            o = o * 1.1
        else:
            o = o * 1.03
    with pytest.raises(AssertionError):
        check_fp8_output(o, lse, q, k, v, sc, causal)


def test_check_rejects_wrong_lse_and_nonzero_empty_rows():
    q, k, v = _inputs(True)
    sc = 1.0 / math.sqrt(D)
    o, lse = _rounded_like_the_kernel(q, k, v, sc, True)
    with pytest.raises(AssertionError, match="LSE"):
        check_fp8_output(o, lse + 2e-3, q, k, v, sc, True)
    # More queries than keys under the causal mask: the first rows see nothing.
    qq = np.concatenate([q, q[:, :, :100]], axis=2)
    o2, lse2 = orc.attention_fwd(qq, k, v, sc, True)
    check_fp8_output(o2, lse2, qq, k, v, sc, True)
    o2[0, 0, 3, 5] = 1e-3
    with pytest.raises(AssertionError, match="without keys"):
        check_fp8_output(o2, lse2, qq, k, v, sc, True)
