"""GPU parity of packed (variable-length) batches against the float64 oracle.

A packed batch concatenates each sequence's dense [H, n_b, d] block; the
oracle splits it and applies the dense definition to each sequence.
"""

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


def run_packed(q, k, v, do, cu_q, cu_k, hq, hkv, causal, max_q=None, max_k=None, out_fill=None):
    """Forward then backward of a packed batch on the GPU; returns CPU tensors."""
    fa = _fa()
    lq = (cu_q[1:] - cu_q[:-1]).tolist()
    lk = (cu_k[1:] - cu_k[:-1]).tolist()
    mq = max(lq) if max_q is None else max_q
    mk = max(lk) if max_k is None else max_k
    qd, kd, vd, dod, cqd, ckd = (dev(t) for t in (q, k, v, do, cu_q, cu_k))
    o = lse = dq = dk = dv = None
    if out_fill is not None:
        o = torch.full_like(qd, out_fill)
        lse = torch.full((qd.shape[0],), out_fill, dtype=torch.float32, device="cuda")
        dq, dk, dv = torch.full_like(qd, out_fill), torch.full_like(kd, out_fill), torch.full_like(vd, out_fill)
    o, lse = fa.fwd_varlen(qd, kd, vd, cqd, ckd, hq, hkv, mq, mk, causal=causal, out=o, lse=lse)
    dq, dk, dv = fa.bwd_varlen(qd, kd, vd, o, dod, lse, cqd, ckd, hq, hkv, mq, mk, causal=causal, dq=dq, dk=dk,
                               dv=dv)
    torch.cuda.synchronize()
    return tuple(t.cpu() for t in (o, lse, dq, dk, dv))


def check_packed(q, k, v, do, cu_q, cu_k, hq, hkv, causal, dtype):
    o, lse, dq, dk, dv = run_packed(q, k, v, do, cu_q, cu_k, hq, hkv, causal)
    sc = scale_for(q.shape[-1])
    ro, rl = orc.attention_fwd_packed(f64(q), f64(k), f64(v), cu_q.numpy(), cu_k.numpy(), hq, hkv, sc, causal)
    rq, rk, rv = orc.attention_bwd_packed(f64(q), f64(k), f64(v), f64(do), cu_q.numpy(), cu_k.numpy(), hq, hkv, sc,
                                          causal)
    assert_close("O", f64(o), ro, dtype, "o")
    assert_close("LSE", f64(lse), rl, dtype, "lse")
    assert_close("dQ", f64(dq), rq, dtype, "grad")
    assert_close("dK", f64(dk), rk, dtype, "grad")
    assert_close("dV", f64(dv), rv, dtype, "grad")


# query lengths, key lengths, Hq, Hkv, d, dtype, causal
CASES = [
    ([128, 77, 300], [128, 77, 300], 2, 2, 64, "bf16", True),
    ([1, 200, 0, 513], [1, 200, 0, 513], 4, 2, 128, "f16", False),
    ([100, 257], [300, 64], 2, 1, 32, "bf16", True),        # Nq < Nk and Nq > Nk (rows without keys)
    ([50, 0, 70], [0, 30, 90], 2, 2, 64, "f16", True),      # queries without keys, keys without queries
    ([50, 0, 70], [0, 30, 90], 2, 2, 64, "f16", False),
    ([33, 130], [33, 130], 1, 1, 32, "f32", False),
    ([129, 64, 17], [129, 64, 17], 2, 2, 128, "f32", True),
    ([700, 17, 1000], [700, 17, 1000], 8, 2, 128, "bf16", True),
    ([255, 256, 257, 1], [255, 256, 257, 1], 3, 3, 64, "bf16", False),
    # 8-wave forward work-groups (B * Hq * 2 tiles of the longest >= 512)
    ([300, 257, 100], [300, 257, 100], 128, 64, 128, "bf16", True),
]


@pytest.mark.parametrize("lens_q,lens_k,hq,hkv,d,dtype,causal", CASES,
                         ids=[f"{len(c[0])}seq_{c[2]}x{c[3]}_d{c[4]}_{c[5]}_{'c' if c[6] else 'nc'}_{i}"
                              for i, c in enumerate(CASES)])
def test_varlen_matches_oracle(lens_q, lens_k, hq, hkv, d, dtype, causal):
    print(f"varlen case lens_q={lens_q} lens_k={lens_k} H={hq}x{hkv} d={d} {dtype} causal={causal}", flush=True)
    q, k, v, do, cu_q, cu_k = si.make_packed_inputs(lens_q, lens_k, hq, hkv, d, dtype,
                                                    seed=5000 + sum(lens_q) + 7 * sum(lens_k) + d)
    check_packed(q, k, v, do, cu_q, cu_k, hq, hkv, causal, dtype)


@pytest.mark.parametrize("causal", [True, False])
def test_varlen_equal_lengths_equal_dense_bitwise(causal):
    """A dense [B, H, N, d] tensor is already a packed batch with cu = [0, N,
    2N, ...]: the packed calls must give bitwise the dense calls' results."""
    fa = _fa()
    B, Hq, Hkv, N, d = 3, 4, 2, 333, 128
    q, k, v, do = si.make_attention_inputs(B, Hq, Hkv, N, N, d, "bf16", seed=91)
    qd, kd, vd, dod = dev(q), dev(k), dev(v), dev(do)
    o, lse = fa.fwd(qd, kd, vd, causal=causal)
    g = fa.bwd(qd, kd, vd, o, dod, lse, causal=causal)
    cu = torch.arange(0, (B + 1) * N, N, dtype=torch.int32, device="cuda")
    flat = lambda t: t.view(-1, d)
    po, pl = fa.fwd_varlen(flat(qd), flat(kd), flat(vd), cu, cu, Hq, Hkv, N, N, causal=causal)
    pg = fa.bwd_varlen(flat(qd), flat(kd), flat(vd), po, flat(dod), pl, cu, cu, Hq, Hkv, N, N, causal=causal)
    torch.cuda.synchronize()
    assert torch.equal(po, flat(o)) and torch.equal(pl, lse.view(-1))
    for a, b in zip(pg, g):
        assert torch.equal(a, flat(b))


def test_varlen_sequence_longer_than_bound_is_skipped():
    """Sequence 1 (200 tokens) exceeds max_seqlen = 150: its rows are left
    unwritten, sequence 0 is computed as usual."""
    hq, hkv, d = 2, 2, 64
    q, k, v, do, cu_q, cu_k = si.make_packed_inputs([100, 200], [100, 200], hq, hkv, d, "bf16", seed=92)
    o, lse, dq, dk, dv = run_packed(q, k, v, do, cu_q, cu_k, hq, hkv, True, max_q=150, max_k=150,
                                    out_fill=float("nan"))
    n0 = hq * 100
    sc = scale_for(d)
    ro, rl = orc.attention_fwd_packed(f64(q[:n0]), f64(k[:n0]), f64(v[:n0]), [0, 100], [0, 100], hq, hkv, sc, True)
    rq, rk, rv = orc.attention_bwd_packed(f64(q[:n0]), f64(k[:n0]), f64(v[:n0]), f64(do[:n0]), [0, 100], [0, 100],
                                          hq, hkv, sc, True)
    assert_close("O", f64(o[:n0]), ro, "bf16", "o")
    assert_close("LSE", f64(lse[:n0]), rl, "bf16", "lse")
    assert_close("dQ", f64(dq[:n0]), rq, "bf16", "grad")
    assert_close("dK", f64(dk[:n0]), rk, "bf16", "grad")
    assert_close("dV", f64(dv[:n0]), rv, "bf16", "grad")
    for name, t in (("O", o), ("LSE", lse), ("dQ", dq), ("dK", dk), ("dV", dv)):
        assert torch.isnan(t[n0:].float()).all(), f"{name}: rows of the skipped sequence were written"


def test_varlen_workload_varlen_bf16():
    """The packed training workload at full size: every sequence is checked
    against the oracle on one of its heads (forward and backward)."""
    w = si.WORKLOADS["varlen_bf16"]
    q, k, v, do, cu_q, cu_k = si.workload_packed_inputs(w)
    print(f"varlen_bf16 lengths {(cu_q[1:] - cu_q[:-1]).tolist()}", flush=True)
    o, lse, dq, dk, dv = run_packed(q, k, v, do, cu_q, cu_k, w.Hq, w.Hkv, w.causal)
    for b in range(w.B):
        n = int(cu_q[b + 1] - cu_q[b])
        h = b % w.Hq
        r0 = w.Hq * int(cu_q[b]) + h * n
        sl = slice(r0, r0 + n)
        sh = lambda t: f64(t[sl]).reshape(1, 1, n, w.d)
        ro, rl = orc.attention_fwd(sh(q), sh(k), sh(v), w.scale, w.causal)
        rq, rk, rv = orc.attention_bwd(sh(q), sh(k), sh(v), sh(do), w.scale, w.causal)
        tag = f"[seq {b}, head {h}, n {n}]"
        assert_close("O" + tag, sh(o), ro, w.dtype, "o")
        assert_close("LSE" + tag, f64(lse[sl]).reshape(1, 1, n), rl, w.dtype, "lse")
        assert_close("dQ" + tag, sh(dq), rq, w.dtype, "grad")
        assert_close("dK" + tag, sh(dk), rk, w.dtype, "grad")
        assert_close("dV" + tag, sh(dv), rv, w.dtype, "grad")
    assert np.isfinite(f64(dq)).all() and np.isfinite(f64(dk)).all() and np.isfinite(f64(dv)).all()
