"""CPU tests of the large-logit O bound (parity.assert_o_within_rounding): it
accepts an output carrying exactly the two bfloat16 roundings the forward
makes, and rejects outputs with planted mistakes.

The accepted output is built here from the oracle's scores: each row's
x = exp(s - max) is rounded to bfloat16 (torch's cast, round to nearest
even), O = sum_j x_j V_j / sum_j x_j (the unrounded sum), and O is rounded to
bfloat16.  The inputs have the large-logit workload's distribution (Q, K
drawn N(0,1) times 8, V N(0,1)), at a size the oracle handles in a second.
"""

from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import synth_inputs as si
from oracle import attention_f64 as orc
from parity import assert_o_within_rounding

N, D = 768, 128


def _inputs():
    q, k, v, _ = si.make_attention_inputs(1, 1, 1, N, N, D, "bf16", seed=4713, qk_mult=8.0)
    return q[0, 0].double().numpy(), k[0, 0].double().numpy(), v[0, 0].double().numpy()


def _rounded_like_the_kernel(q, k, v, scale):
    s = scale * (q @ k.T)
    vis = orc.visible_mask(N, N, True)
    s = np.where(vis, s, -np.inf)
    x = np.where(vis, np.exp(s - s.max(axis=1, keepdims=True)), 0.0)
    xr = torch.from_numpy(x).float().to(torch.bfloat16).double().numpy()
    o = (xr @ v) / x.sum(axis=1, keepdims=True)
    return torch.from_numpy(o).to(torch.bfloat16).double().numpy()


def test_bound_accepts_bf16_rounded_output():
    q, k, v = _inputs()
    sc = 1.0 / math.sqrt(D)
    o = _rounded_like_the_kernel(q, k, v, sc)
    err, rms, ratio = assert_o_within_rounding("O", o, q, k, v, sc, True)
    assert rms < 0.9 and ratio < 1.0


@pytest.mark.parametrize("mistake", ["scaled by 1.03", "rows past 256 halved", "one key dropped",
                                     "top-left mask"])
def test_bound_rejects_planted_mistake(mistake):
    q, k, v = _inputs()
    sc = 1.0 / math.sqrt(D)
    o = _rounded_like_the_kernel(q, k, v, sc)
    if mistake == "scaled by 1.03":
        o = o * 1.03
    elif mistake == "rows past 256 halved":
        o[256:] *= 0.5
    elif mistake == "one key dropped":
        p, _ = orc.attention_probs(q, k, sc, True)
        o = o - np.outer(p[:, 100], v[100])
    else:
        # keys beyond the row for a query sequence shifted by 64 rows
        p, _ = orc.attention_probs(q, k, sc, True, row_ids=np.arange(N) + 64, nq_total=N)
        o = p @ v
    with pytest.raises(AssertionError):
        assert_o_within_rounding("O", o, q, k, v, sc, True)
