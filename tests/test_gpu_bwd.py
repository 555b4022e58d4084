"""GPU parity of the backward kernels against the float64 oracle's gradients."""

from __future__ import annotations

import numpy as np
import pytest
import torch

from parity import assert_close, dev, f64, scale_for
from oracle import attention_f64 as orc
import synth_inputs as si

pytestmark = pytest.mark.gpu


def _fa():
    import exact_io_aware_47_amd as fa
    return fa


def run_fwd_bwd(q, k, v, do, causal, scale=None):
    """Forward then backward on the GPU (the backward consumes the kernel's own O and LSE)."""
    fa = _fa()
    qd, kd, vd, dod = dev(q), dev(k), dev(v), dev(do)
    o, lse = fa.fwd(qd, kd, vd, causal=causal, scale=scale)
    dq, dk, dv = fa.bwd(qd, kd, vd, o, dod, lse, causal=causal, scale=scale)
    torch.cuda.synchronize()
    return dq.cpu(), dk.cpu(), dv.cpu()


def check_grads(q, k, v, do, causal, dtype, scale=None, large_logits=False):
    sc = scale_for(q.shape[-1]) if scale is None else scale
    dq, dk, dv = run_fwd_bwd(q, k, v, do, causal, scale)
    rq, rk, rv = orc.attention_bwd(f64(q), f64(k), f64(v), f64(do), sc, causal)
    assert_close("dQ", f64(dq), rq, dtype, "grad", large_logits)
    assert_close("dK", f64(dk), rk, dtype, "grad", large_logits)
    assert_close("dV", f64(dv), rv, dtype, "grad", large_logits)


# B, Hq, Hkv, Nq, Nk, d, dtype, causal
CASES = [
    (1, 1, 1, 128, 128, 32, "f32", False),
    (1, 2, 2, 77, 77, 32, "f32", True),
    (1, 2, 1, 150, 250, 64, "f32", False),
    (1, 2, 2, 129, 129, 128, "f32", True),
    (1, 2, 2, 1, 1, 64, "bf16", False),
    (2, 4, 4, 257, 257, 64, "f16", True),
    (1, 4, 1, 300, 513, 128, "bf16", True),
    (1, 4, 2, 513, 300, 128, "bf16", True),
    (1, 2, 2, 100, 300, 32, "f16", True),
    (2, 8, 8, 600, 600, 128, "bf16", False),
    (1, 8, 2, 384, 384, 32, "f16", False),
    (1, 2, 2, 64, 64, 128, "f16", True),
    (3, 6, 3, 190, 190, 128, "f16", False),
    (1, 6, 2, 1000, 1000, 64, "bf16", True),
    # causal with keys far beyond the queries (most key tiles need no mask),
    # with more queries than keys, and with GQA over an offset diagonal
    (1, 2, 2, 64, 1000, 128, "bf16", True),
    (2, 4, 2, 700, 256, 64, "bf16", True),
    (1, 3, 1, 200, 700, 128, "f16", True),
    # bfloat16 at d = 32
    (2, 4, 4, 333, 333, 32, "bf16", True),
    (1, 3, 1, 200, 517, 32, "bf16", False),
    # many heads of short sequences (the forward runs 8-wave work-groups)
    (2, 256, 64, 257, 300, 64, "bf16", True),
    (2, 128, 128, 300, 257, 128, "f16", False),
]


@pytest.mark.parametrize("B,Hq,Hkv,Nq,Nk,d,dtype,causal", CASES,
                         ids=[f"B{c[0]}_H{c[1]}x{c[2]}_N{c[3]}x{c[4]}_d{c[5]}_{c[6]}_{'c' if c[7] else 'nc'}" for c in CASES])
def test_bwd_matches_oracle(B, Hq, Hkv, Nq, Nk, d, dtype, causal):
    q, k, v, do = si.make_attention_inputs(B, Hq, Hkv, Nq, Nk, d, dtype, seed=2000 + Nq + 3 * Nk + d)
    check_grads(q, k, v, do, causal, dtype)


def test_bwd_unusual_scale():
    q, k, v, do = si.make_attention_inputs(1, 2, 2, 150, 150, 64, "bf16", seed=78)
    for scale in (0.0, -0.3):
        for causal in (False, True):
            check_grads(q, k, v, do, causal, "bf16", scale=scale)


def test_bwd_workload_mha_f32_small():
    w = si.WORKLOADS["mha_f32_small"]
    q, k, v, do = si.workload_attention_inputs(w)
    check_grads(q, k, v, do, False, "f32")


@pytest.mark.parametrize("causal", [True, False])
def test_bwd_workload_mha_f16(causal):
    w = si.WORKLOADS["mha_f16"]
    q, k, v, do = si.workload_attention_inputs(w)
    check_grads(q, k, v, do, causal, "f16")


def _oracle_bwd_rows(q, k, v, do, scale, causal, chunk):
    """The oracle's gradients of one (batch, head), taking the query rows in
    chunks: dQ rows come from their own chunk, dK and dV sum the chunks'
    contributions (each row's terms depend on that row alone)."""
    nq = q.shape[2]
    dq = np.zeros(q.shape)
    dk = np.zeros(k.shape)
    dv = np.zeros(v.shape)
    for r0 in range(0, nq, chunk):
        rows = np.arange(r0, min(r0 + chunk, nq))
        gq, gk, gv = orc.attention_bwd(q[:, :, rows], k, v, do[:, :, rows], scale, causal, row_ids=rows, nq_total=nq)
        dq[:, :, rows] = gq
        dk += gk
        dv += gv
    return dq, dk, dv


def _heads_check(w, heads, chunk=None):
    q, k, v, do = si.workload_attention_inputs(w)
    dq, dk, dv = run_fwd_bwd(q, k, v, do, True)
    large = w.qk_mult != 1.0
    for b, h in heads:
        sl = (slice(b, b + 1), slice(h, h + 1))
        if chunk is None:
            rq, rk, rv = orc.attention_bwd(f64(q[sl]), f64(k[sl]), f64(v[sl]), f64(do[sl]), w.scale, True)
        else:
            rq, rk, rv = _oracle_bwd_rows(f64(q[sl]), f64(k[sl]), f64(v[sl]), f64(do[sl]), w.scale, True, chunk)
        assert_close(f"dQ[{b},{h}]", f64(dq[sl]), rq, w.dtype, "grad", large)
        assert_close(f"dK[{b},{h}]", f64(dk[sl]), rk, w.dtype, "grad", large)
        assert_close(f"dV[{b},{h}]", f64(dv[sl]), rv, w.dtype, "grad", large)
    return dq, dk, dv


def test_bwd_workload_mha_bf16_4k():
    """The benchmarked launch, compared in full (every head)."""
    w = si.WORKLOADS["mha_bf16_4k"]
    _heads_check(w, [(b, h) for b in range(w.B) for h in range(w.Hq)])


def test_bwd_workload_gqa_bf16_4k():
    """Grouped heads at the training shape: dK/dV of one K/V head are the sum
    over its four query heads, so the oracle takes whole groups (three of
    them, the last included)."""
    w = si.WORKLOADS["gqa_bf16_4k"]
    q, k, v, do = si.workload_attention_inputs(w)
    dq, dk, dv = run_fwd_bwd(q, k, v, do, True)
    g = w.Hq // w.Hkv
    for b, hkv in ((0, 0), (1, 5), (1, w.Hkv - 1)):
        qs = (slice(b, b + 1), slice(hkv * g, (hkv + 1) * g))
        ks = (slice(b, b + 1), slice(hkv, hkv + 1))
        rq, rk, rv = orc.attention_bwd(f64(q[qs]), f64(k[ks]), f64(v[ks]), f64(do[qs]), w.scale, True)
        assert_close(f"dQ[{b},group {hkv}]", f64(dq[qs]), rq, w.dtype, "grad")
        assert_close(f"dK[{b},{hkv}]", f64(dk[ks]), rk, w.dtype, "grad")
        assert_close(f"dV[{b},{hkv}]", f64(dv[ks]), rv, w.dtype, "grad")


def test_bwd_workload_mha_bf16_16k():
    """Two whole heads, the last included (oracle rows in chunks of 2048)."""
    dq, dk, dv = _heads_check(si.WORKLOADS["mha_bf16_16k"], [(0, 5), (0, 15)], chunk=2048)
    for t in (dq, dk, dv):
        assert torch.isfinite(t.float()).all()


def test_bwd_bitwise_repeatable():
    q, k, v, do = si.make_attention_inputs(1, 4, 2, 700, 700, 128, "bf16", seed=4)
    fa = _fa()
    qd, kd, vd, dod = dev(q), dev(k), dev(v), dev(do)
    o, lse = fa.fwd(qd, kd, vd, causal=True)
    g1 = fa.bwd(qd, kd, vd, o, dod, lse, causal=True)
    g2 = fa.bwd(qd, kd, vd, o, dod, lse, causal=True)
    torch.cuda.synchronize()
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)


def _three_phases(fa, qd, kd, vd, o, dod, lse, ws, causal):
    """Preprocess, dK/dV, dQ in that order on the current stream."""
    dq, dk, dv = torch.empty_like(qd), torch.empty_like(kd), torch.empty_like(vd)
    fa.bwd_phase("preprocess", None, None, None, o, dod, lse, None, None, None, ws, causal)
    fa.bwd_phase("dkdv", qd, kd, vd, None, dod, None, None, dk, dv, ws, causal)
    fa.bwd_phase("dq", qd, kd, vd, None, dod, None, dq, None, None, ws, causal)
    return dq, dk, dv


def test_bwd_phases_on_two_streams_match_single_call():
    """Preprocess, then dK/dV on the current stream and dQ on a second stream
    concurrently: bitwise equal to the three phases in order on one stream."""
    fa = _fa()
    q, k, v, do = si.make_attention_inputs(2, 8, 4, 513, 513, 64, "f16", seed=6)
    qd, kd, vd, dod = dev(q), dev(k), dev(v), dev(do)
    o, lse = fa.fwd(qd, kd, vd, causal=True)
    ws = torch.empty(fa.bwd_workspace_bytes(2, 8, 4, 513, 513, 64, fa.FA_F16), dtype=torch.uint8, device="cuda")
    ref = _three_phases(fa, qd, kd, vd, o, dod, lse, ws, True)
    dq, dk, dv = torch.empty_like(qd), torch.empty_like(kd), torch.empty_like(vd)
    main = torch.cuda.current_stream()
    side = torch.cuda.Stream()
    fa.bwd_phase("preprocess", None, None, None, o, dod, lse, None, None, None, ws, True)
    ready = torch.cuda.Event()
    ready.record(main)
    side.wait_event(ready)
    with torch.cuda.stream(side):
        fa.bwd_phase("dq", qd, kd, vd, None, dod, None, dq, None, None, ws, True)
    fa.bwd_phase("dkdv", qd, kd, vd, None, dod, None, None, dk, dv, ws, True)
    main.wait_stream(side)
    torch.cuda.synchronize()
    for a, b in zip((dq, dk, dv), ref):
        assert torch.equal(a, b)


# B, Hq, Hkv, Nq, Nk, d, dtype, causal: ragged tails, GQA, more queries than
# keys (causal rows that see no key), all three element types.
ROWTERM_CASES = [
    (2, 8, 4, 513, 513, 64, "f16", True),
    (1, 4, 2, 700, 256, 128, "bf16", True),
    (1, 2, 2, 129, 300, 32, "f32", False),
    (2, 4, 1, 333, 333, 128, "bf16", False),
]


@pytest.mark.parametrize("B,Hq,Hkv,Nq,Nk,d,dtype,causal", ROWTERM_CASES,
                         ids=[f"{c[0]}x{c[1]}x{c[2]}_{c[3]}x{c[4]}_d{c[5]}_{c[6]}_{'c' if c[7] else 'nc'}"
                              for c in ROWTERM_CASES])
def test_bwd_is_dq_with_row_terms_then_dkdv(B, Hq, Hkv, Nq, Nk, d, dtype, causal):
    """flash_attn_bwd is the dQ phase that computes the row terms followed by
    dK/dV: bitwise equal to those two phases called in order.  The row terms
    it leaves in the workspace agree with the preprocess kernel's (LSE*log2(e)
    bitwise; D_i within the rounding of a float32 sum of d products), and the
    gradients agree with the three-phase order to the same bound as each has
    with the oracle, which both are checked against."""
    fa = _fa()
    q, k, v, do = si.make_attention_inputs(B, Hq, Hkv, Nq, Nk, d, dtype, seed=11)
    qd, kd, vd, dod = dev(q), dev(k), dev(v), dev(do)
    o, lse = fa.fwd(qd, kd, vd, causal=causal)
    fused = fa.bwd(qd, kd, vd, o, dod, lse, causal=causal)
    code = {"f32": fa.FA_F32, "f16": fa.FA_F16, "bf16": fa.FA_BF16}[dtype]
    nbytes = fa.bwd_workspace_bytes(B, Hq, Hkv, Nq, Nk, d, code)
    ws = torch.full((nbytes,), 0x7F, dtype=torch.uint8, device="cuda")
    dq, dk, dv = torch.empty_like(qd), torch.empty_like(kd), torch.empty_like(vd)
    fa.bwd_phase("dq_rowterms", qd, kd, vd, o, dod, lse, dq, None, None, ws, causal)
    rows = B * Hq * Nq
    terms = ws[: 8 * rows].view(torch.float32).clone()
    fa.bwd_phase("dkdv", qd, kd, vd, None, dod, None, None, dk, dv, ws, causal)
    ws3 = torch.empty_like(ws)
    three = _three_phases(fa, qd, kd, vd, o, dod, lse, ws3, causal)
    terms3 = ws3[: 8 * rows].view(torch.float32).clone()
    torch.cuda.synchronize()
    for a, b in zip((dq, dk, dv), fused):
        assert torch.equal(a, b)
    assert torch.equal(terms[rows:], terms3[rows:])
    dsum, dsum3 = terms[:rows].double(), terms3[:rows].double()
    mag = (dod.double() * o.double()).abs().sum(-1).reshape(-1)
    assert torch.all((dsum - dsum3).abs() <= 2 * d * 2.0 ** -24 * mag + 1e-30)
    sc = scale_for(d)
    rq, rk, rv = orc.attention_bwd(f64(q), f64(k), f64(v), f64(do), sc, causal)
    for name, g, r in (("dQ", dq, rq), ("dK", dk, rk), ("dV", dv, rv)):
        assert_close(name, f64(g.cpu()), r, dtype, "grad")
