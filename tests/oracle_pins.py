"""Pins of the float64 oracle: checks against what the pages and mathematics fix.

Each ``pin_*`` function takes the oracle module as its argument and raises
AssertionError when the oracle disagrees with a value printed on the pages, a
closed form, an invariant of the mathematics, brute force on a tiny input or
an independent library routine (torch's CPU float64 scaled-dot-product
attention and autograd).  ``tests/test_oracle.py`` runs every pin on the real
oracle and, to show that the pins have teeth, on mutated copies of the oracle
with one plausible mistake planted in each (all on the CPU).
"""

from __future__ import annotations

import json
import math
import os

import numpy as np
import torch

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


def _rand(rng, *shape):
    return rng.standard_normal(shape)


def _normwise(x, ref):
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = max(np.abs(ref).max(), 1e-300)
    return np.abs(x - ref).max() / den


# ---------------------------------------------------------------------------
# Online-softmax worked example (tutorial: "Online softmax", "Correction
# formula" and the worked example of the streaming process).
# ---------------------------------------------------------------------------

def _worked_example():
    with open(os.path.join(GOLDEN, "online_softmax_worked_example.json")) as f:
        g = json.load(f)
    pv, ch = g["page_values"], g["chosen"]
    b1 = [pv["block1_max"] + math.log(w) for w in ch["block1_weights"]]
    b2 = [pv["block2_max"] + math.log(w) for w in ch["block2_weights"]]
    return pv, ch, b1, b2


def pin_worked_example_streaming(orc):
    pv, ch, b1, b2 = _worked_example()
    # Block 1 alone: the page's max 2.0 and sum 3.1.
    m1, l1 = orc.online_softmax_stats(b1, block=len(b1))
    assert m1 == pv["block1_max"], m1
    assert abs(l1 - pv["block1_sum"]) < 1e-14, l1
    # Both blocks streamed: max 3.5; old sum rescaled by exp(2.0 - 3.5), plus block 2's sum.
    m, l = orc.online_softmax_stats(b1 + b2, block=len(b1))
    assert m == pv["block2_max"], m
    expect_l = pv["block1_sum"] * math.exp(pv["block1_max"] - pv["block2_max"]) + ch["block2_sum"]
    assert abs(l - expect_l) < 1e-14, (l, expect_l)
    # The merge of the two blocks' separately taken statistics gives the same.
    m2, l2 = orc.online_softmax_stats(b2, block=len(b2))
    mm, lm = orc.merge_softmax_stats(m1, l1, m2, l2)
    assert mm == m and abs(lm - expect_l) < 1e-14, (mm, lm)
    # Every block size gives the two-pass result (the streaming is exact).
    for blk in (1, 2, 3, 5, 6, 100):
        mb, lb = orc.online_softmax_stats(b1 + b2, block=blk)
        assert mb == m and abs(lb - expect_l) < 1e-14, (blk, mb, lb)


def pin_worked_example_attention(orc):
    """The attention forward on a row whose scores are the worked example's six
    values must produce the same normaliser: LSE = 3.5 + ln(total sum)."""
    pv, ch, b1, b2 = _worked_example()
    scores = np.array(b1 + b2)
    # d = 1, q = [1], k_j = [score_j], scale 1: S row = the six scores.
    q = np.ones((1, 1, 1, 1))
    k = scores.reshape(1, 1, -1, 1)
    v = np.eye(len(scores)).reshape(1, 1, len(scores), len(scores))  # O = P
    o, lse = orc.attention_fwd(q, k, v, 1.0, False)
    total = pv["block1_sum"] * math.exp(pv["block1_max"] - pv["block2_max"]) + ch["block2_sum"]
    assert abs(lse[0, 0, 0] - (pv["block2_max"] + math.log(total))) < 1e-14
    weights = np.array([w * math.exp(pv["block1_max"] - pv["block2_max"]) for w in ch["block1_weights"]]
                       + list(ch["block2_weights"])) / total
    assert np.abs(o[0, 0, 0] - weights).max() < 1e-15


# ---------------------------------------------------------------------------
# Softmax normalisation and forward invariants
# ---------------------------------------------------------------------------

def pin_rows_sum_to_one(orc):
    rng = _rng(1)
    for causal, nq, nk in ((False, 7, 9), (True, 9, 9), (True, 5, 11)):
        q, k = _rand(rng, nq, 6), _rand(rng, nk, 6)
        p, _ = orc.attention_probs(q, k, 0.4, causal)
        assert (p >= 0).all()
        assert np.abs(p.sum(axis=1) - 1.0).max() < 1e-15
        if causal:
            mask = np.arange(nk)[None, :] <= (np.arange(nq) + nk - nq)[:, None]
            assert (p[~mask] == 0).all()
            assert (p[mask] > 0).all()


def pin_constant_v(orc):
    rng = _rng(2)
    for causal in (False, True):
        q, k = _rand(rng, 2, 3, 12, 8), _rand(rng, 2, 1, 12, 8)
        vrow = _rand(rng, 8)
        v = np.broadcast_to(vrow, (2, 1, 12, 8)).copy()
        o, _ = orc.attention_fwd(q, k, v, 0.3, causal)
        assert np.abs(o - vrow).max() < 1e-14


def pin_key_permutation(orc):
    rng = _rng(3)
    q, k, v = _rand(rng, 1, 2, 6, 5), _rand(rng, 1, 2, 10, 5), _rand(rng, 1, 2, 10, 4)
    o, lse = orc.attention_fwd(q, k, v, 0.7, False)
    perm = rng.permutation(10)
    o2, lse2 = orc.attention_fwd(q, k[:, :, perm], v[:, :, perm], 0.7, False)
    assert np.abs(o - o2).max() < 1e-14 and np.abs(lse - lse2).max() < 1e-13


def pin_key_translation(orc):
    """K <- K + 1 uᵀ adds scale * q_i·u to every score of row i: O unchanged,
    LSE_i shifted by exactly that amount (causal rows too)."""
    rng = _rng(4)
    for causal in (False, True):
        q, k, v = _rand(rng, 1, 1, 8, 6), _rand(rng, 1, 1, 8, 6), _rand(rng, 1, 1, 8, 6)
        u = _rand(rng, 6)
        o, lse = orc.attention_fwd(q, k, v, 0.5, causal)
        o2, lse2 = orc.attention_fwd(q, k + u, v, 0.5, causal)
        assert np.abs(o - o2).max() < 1e-13
        shift = 0.5 * (q[0, 0] @ u)
        assert np.abs(lse2[0, 0] - lse[0, 0] - shift).max() < 1e-12


def pin_zero_query_closed_form(orc):
    """Q = 0 makes every visible score 0: P uniform over the visible keys."""
    rng = _rng(5)
    for causal, nq, nk in ((False, 6, 9), (True, 9, 9), (True, 4, 9)):
        v = _rand(rng, 1, 1, nk, 5)
        q = np.zeros((1, 1, nq, 5))
        k = _rand(rng, 1, 1, nk, 5)
        o, lse = orc.attention_fwd(q, k, v, 0.9, causal)
        for i in range(nq):
            n_vis = nk if not causal else i + 1 + nk - nq
            assert np.abs(o[0, 0, i] - v[0, 0, :n_vis].mean(axis=0)).max() < 1e-14
            assert abs(lse[0, 0, i] - math.log(n_vis)) < 1e-14


def pin_single_key(orc):
    """Nk = 1: O = V_0, LSE = scale q·k_0, dQ = dK = 0, dV = Σ_i dO_i."""
    rng = _rng(6)
    q, k, v, do = _rand(rng, 1, 2, 5, 4), _rand(rng, 1, 2, 1, 4), _rand(rng, 1, 2, 1, 4), _rand(rng, 1, 2, 5, 4)
    o, lse = orc.attention_fwd(q, k, v, 0.25, False)
    assert np.abs(o - v).max() == 0.0
    assert np.abs(lse - 0.25 * np.einsum("bhid,bhd->bhi", q, k[:, :, 0])).max() < 1e-14
    dq, dk, dv = orc.attention_bwd(q, k, v, do, 0.25, False)
    assert np.abs(dq).max() < 1e-15 and np.abs(dk).max() < 1e-14
    assert np.abs(dv[:, :, 0] - do.sum(axis=2)).max() < 1e-14


def pin_causal_first_row(orc):
    rng = _rng(7)
    q, k, v = _rand(rng, 1, 1, 6, 4), _rand(rng, 1, 1, 6, 4), _rand(rng, 1, 1, 6, 4)
    o, lse = orc.attention_fwd(q, k, v, 0.5, True)
    assert np.array_equal(o[0, 0, 0], v[0, 0, 0])
    assert abs(lse[0, 0, 0] - 0.5 * q[0, 0, 0] @ k[0, 0, 0]) < 1e-14


def pin_fully_masked_rows(orc):
    """Causal with Nq > Nk: the first Nq - Nk rows see no key (bottom-right)."""
    rng = _rng(8)
    q, k, v, do = _rand(rng, 1, 1, 7, 3), _rand(rng, 1, 1, 4, 3), _rand(rng, 1, 1, 4, 3), _rand(rng, 1, 1, 7, 3)
    o, lse = orc.attention_fwd(q, k, v, 0.5, True)
    assert (o[0, 0, :3] == 0).all() and np.isneginf(lse[0, 0, :3]).all()
    assert np.isfinite(lse[0, 0, 3:]).all()
    assert np.array_equal(o[0, 0, 3], v[0, 0, 0])
    dq, dk, dv = orc.attention_bwd(q, k, v, do, 0.5, True)
    assert (dq[0, 0, :3] == 0).all()
    assert np.isfinite(dq).all() and np.isfinite(dk).all() and np.isfinite(dv).all()


# ---------------------------------------------------------------------------
# Independent library routine: torch CPU float64 SDPA + autograd
# ---------------------------------------------------------------------------

def _torch_reference(q, k, v, do, scale, causal):
    tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    g = q.shape[1] // k.shape[1]
    nq, nk = q.shape[2], k.shape[2]
    mask = None
    if causal:
        mask = torch.ones(nq, nk, dtype=torch.bool).tril(diagonal=nk - nq)
    out = torch.nn.functional.scaled_dot_product_attention(
        tq, tk.repeat_interleave(g, dim=1), tv.repeat_interleave(g, dim=1), attn_mask=mask, scale=scale)
    out.backward(torch.tensor(do, dtype=torch.float64))
    scores = scale * tq.detach() @ tk.detach().repeat_interleave(g, dim=1).transpose(-1, -2)
    if causal:
        scores = scores.masked_fill(~mask, -math.inf)
    lse = torch.logsumexp(scores, dim=-1)
    return (out.detach().numpy(), lse.numpy(), tq.grad.numpy(), tk.grad.numpy(), tv.grad.numpy())


def pin_matches_torch_cpu_f64(orc):
    rng = _rng(9)
    cases = [
        (2, 4, 4, 33, 33, 16, False),
        (1, 4, 2, 40, 40, 8, True),
        (1, 6, 1, 17, 29, 8, True),  # Nq < Nk causal, MQA
        (2, 2, 2, 29, 17, 4, False),
    ]
    for b, hq, hkv, nq, nk, d, causal in cases:
        q, k, v = _rand(rng, b, hq, nq, d), _rand(rng, b, hkv, nk, d), _rand(rng, b, hkv, nk, d)
        do = _rand(rng, b, hq, nq, d)
        scale = 1.0 / math.sqrt(d)
        o, lse = orc.attention_fwd(q, k, v, scale, causal)
        dq, dk, dv = orc.attention_bwd(q, k, v, do, scale, causal)
        to, tlse, tdq, tdk, tdv = _torch_reference(q, k, v, do, scale, causal)
        assert _normwise(o, to) < 1e-13, "O"
        assert np.abs(lse - tlse).max() < 1e-12, "LSE"
        assert _normwise(dq, tdq) < 1e-12, "dQ"
        assert _normwise(dk, tdk) < 1e-12, "dK"
        assert _normwise(dv, tdv) < 1e-12, "dV"


# ---------------------------------------------------------------------------
# Backward: brute force (central finite differences) and invariants
# ---------------------------------------------------------------------------

def _loss(orc, q, k, v, do, scale, causal):
    o, _ = orc.attention_fwd(q, k, v, scale, causal)
    return float((o * do).sum())


def pin_finite_differences(orc):
    rng = _rng(10)
    h = 1e-6
    for nq, nk, d, causal in ((1, 3, 2, False), (3, 5, 4, True), (5, 3, 2, False),
                              (5, 5, 4, True), (3, 1, 2, True), (5, 3, 4, True)):
        q, k, v = _rand(rng, 1, 2, nq, d), _rand(rng, 1, 1, nk, d), _rand(rng, 1, 1, nk, d)
        do = _rand(rng, 1, 2, nq, d)
        scale = 0.6
        grads = orc.attention_bwd(q, k, v, do, scale, causal)
        for x_idx, g in zip(range(3), grads):
            fd = np.zeros_like(g)
            for idx in np.ndindex(*g.shape):
                args = [q.copy(), k.copy(), v.copy()]
                args[x_idx][idx] += h
                up = _loss(orc, *args, do, scale, causal)
                args[x_idx][idx] -= 2 * h
                dn = _loss(orc, *args, do, scale, causal)
                fd[idx] = (up - dn) / (2 * h)
            den = max(np.abs(fd).max(), 1e-3)
            assert np.abs(g - fd).max() / den < 1e-7, (nq, nk, d, causal, x_idx)


def pin_backward_invariants(orc):
    rng = _rng(11)
    for causal in (False, True):
        q, k, v, do = _rand(rng, 1, 2, 9, 6), _rand(rng, 1, 2, 9, 6), _rand(rng, 1, 2, 9, 5), _rand(rng, 1, 2, 9, 5)
        dq, dk, dv = orc.attention_bwd(q, k, v, do, 0.4, causal)
        # Every row of dS sums to zero, so Σ_j dK_j = scale Σ_ij dS_ij q_i = 0.
        assert np.abs(dk.sum(axis=2)).max() < 1e-13
        # Rows of P sum to one, so Σ_j dV_j = Σ_i dO_i.
        assert np.abs(dv.sum(axis=2) - do.sum(axis=2)).max() < 1e-13


def pin_gqa_equals_repeated_mha(orc):
    rng = _rng(12)
    for causal in (False, True):
        hq, hkv = 6, 2
        q, k, v = _rand(rng, 2, hq, 7, 4), _rand(rng, 2, hkv, 7, 4), _rand(rng, 2, hkv, 7, 4)
        do = _rand(rng, 2, hq, 7, 4)
        g = hq // hkv
        kr, vr = np.repeat(k, g, axis=1), np.repeat(v, g, axis=1)
        o, lse = orc.attention_fwd(q, k, v, 0.5, causal)
        o2, lse2 = orc.attention_fwd(q, kr, vr, 0.5, causal)
        assert np.abs(o - o2).max() == 0 and np.abs(lse - lse2).max() == 0
        dq, dk, dv = orc.attention_bwd(q, k, v, do, 0.5, causal)
        dq2, dk2, dv2 = orc.attention_bwd(q, kr, vr, do, 0.5, causal)
        assert np.abs(dq - dq2).max() == 0
        assert np.abs(dk - dk2.reshape(2, hkv, g, 7, 4).sum(axis=2)).max() < 1e-14
        assert np.abs(dv - dv2.reshape(2, hkv, g, 7, 4).sum(axis=2)).max() < 1e-14


def pin_row_subset(orc):
    """Evaluating a subset of query rows (with their causal horizon) equals
    the same rows of the full evaluation."""
    rng = _rng(13)
    q, k, v, do = _rand(rng, 1, 2, 12, 4), _rand(rng, 1, 1, 15, 4), _rand(rng, 1, 1, 15, 4), _rand(rng, 1, 2, 12, 4)
    rows = np.array([0, 3, 7, 11])
    for causal in (False, True):
        o, lse = orc.attention_fwd(q, k, v, 0.5, causal)
        o2, lse2 = orc.attention_fwd(q[:, :, rows], k, v, 0.5, causal, row_ids=rows, nq_total=12)
        assert np.array_equal(o[:, :, rows], o2) and np.array_equal(lse[:, :, rows], lse2)


# ---------------------------------------------------------------------------
# Paged decode
# ---------------------------------------------------------------------------

def _paged_case(rng, b, hq, hkv, lens, d, bs, extra=3):
    max_blocks = max(1, -(-max(lens) // bs))
    nblk = b * max_blocks + extra
    kc, vc = _rand(rng, nblk, hkv, bs, d), _rand(rng, nblk, hkv, bs, d)
    table = rng.permutation(nblk)[: b * max_blocks].reshape(b, max_blocks)
    q = _rand(rng, b, hq, d)
    return q, kc, vc, table, np.array(lens)


def pin_paged_decode_equals_contiguous(orc):
    rng = _rng(14)
    bs = 4
    q, kc, vc, table, lens = _paged_case(rng, 3, 4, 2, [13, 1, 8], 5, bs)
    o, lse = orc.decode_paged(q, kc, vc, table, lens, 0.45)
    for b in range(3):
        n = lens[b]
        # Independent gather: token t -> (page table[t // bs], slot t % bs), element by element.
        kb = np.zeros((2, n, 5))
        vb = np.zeros((2, n, 5))
        for t in range(n):
            kb[:, t] = kc[table[b, t // bs], :, t % bs]
            vb[:, t] = vc[table[b, t // bs], :, t % bs]
        o_ref, lse_ref = orc.attention_fwd(q[b][None, :, None, :], kb[None], vb[None], 0.45, False)
        assert np.abs(o[b] - o_ref[0, :, 0]).max() < 1e-15
        assert np.abs(lse[b] - lse_ref[0, :, 0]).max() < 1e-15


def pin_paged_decode_table_permutation(orc):
    """Moving pages to other cache slots (and updating the table) changes nothing."""
    rng = _rng(15)
    q, kc, vc, table, lens = _paged_case(rng, 2, 4, 4, [10, 7], 3, 4)
    o, lse = orc.decode_paged(q, kc, vc, table, lens, 0.5)
    perm = rng.permutation(kc.shape[0])  # new slot of old page p is perm[p]
    kc2, vc2 = np.empty_like(kc), np.empty_like(vc)
    kc2[perm], vc2[perm] = kc, vc
    o2, lse2 = orc.decode_paged(q, kc2, vc2, perm[table], lens, 0.5)
    assert np.array_equal(o, o2) and np.array_equal(lse, lse2)


def pin_decode_empty_sequence(orc):
    rng = _rng(16)
    q, kc, vc, table, lens = _paged_case(rng, 2, 2, 1, [0, 5], 3, 4)
    o, lse = orc.decode_paged(q, kc, vc, table, lens, 0.5)
    assert (o[0] == 0).all() and np.isneginf(lse[0]).all() and np.isfinite(lse[1]).all()


def _scatter_to_pages(rng, k, bs, extra=2):
    """Independent paging of a contiguous [B, Hkv, n, d] tensor: a random table
    and a cache whose page table[b, t // bs], slot t % bs holds token t."""
    b, hkv, n, d = k.shape
    max_blocks = -(-n // bs)
    nblk = b * max_blocks + extra
    table = rng.permutation(nblk)[: b * max_blocks].reshape(b, max_blocks)
    cache = _rand(rng, nblk, hkv, bs, d)  # unused slots hold noise
    for bi in range(b):
        for t in range(n):
            cache[table[bi, t // bs], :, t % bs] = k[bi, :, t]
    return cache, table


def pin_prefill_paged_equals_contiguous(orc):
    """A chunk of queries over pages equals the dense definition over the same
    keys stored contiguously, masked bottom-right (queries are the last
    positions); sequences shorter than the cache rows ignore the rest."""
    rng = _rng(18)
    bs, hq, hkv, d = 4, 4, 2, 3
    for nq, n, causal in ((5, 13, True), (5, 13, False), (1, 9, True), (6, 6, True), (7, 3, True)):
        k, v = _rand(rng, 2, hkv, n, d), _rand(rng, 2, hkv, n, d)
        q = _rand(rng, 2, hq, nq, d)
        kc, table = _scatter_to_pages(rng, k, bs)
        vc = np.zeros_like(kc)
        for bi in range(2):
            for t in range(n):
                vc[table[bi, t // bs], :, t % bs] = v[bi, :, t]
        o, lse = orc.prefill_paged(q, kc, vc, table, [n, n], 0.55, causal)
        o_ref, lse_ref = orc.attention_fwd(q, k, v, 0.55, causal)
        assert np.array_equal(np.isinf(lse), np.isinf(lse_ref))
        assert np.abs(o - o_ref).max() < 1e-14
        fin = np.isfinite(lse_ref)
        assert np.abs(lse[fin] - lse_ref[fin]).max() < 1e-14
        if causal and nq <= n:
            # the chunk's last query sees every key, its first sees n - nq + 1
            p_last, _ = orc.attention_probs(q[0, 0], k[0, 0], 0.55, False)
            assert np.abs(o[0, 0, -1] - (p_last @ v[0, 0])[-1]).max() < 1e-14
        # a shorter second sequence reads only its own first tokens
        o2, _ = orc.prefill_paged(q, kc, vc, table, [n, n - 1], 0.55, causal)
        o2_ref, _ = orc.attention_fwd(q[1:], k[1:, :, : n - 1], v[1:, :, : n - 1], 0.55, causal)
        assert np.abs(o2[1] - o2_ref[0]).max() < 1e-14 and np.array_equal(o2[0], o[0])


def pin_prefill_one_query_is_decode(orc):
    """With one query per sequence, prefill over pages is the paged decode
    (the single query is the last position, so the causal mask hides nothing)."""
    rng = _rng(19)
    q, kc, vc, table, lens = _paged_case(rng, 3, 4, 2, [13, 1, 8], 5, 4)
    o_d, lse_d = orc.decode_paged(q, kc, vc, table, lens, 0.45)
    for causal in (False, True):
        o, lse = orc.prefill_paged(q[:, :, None, :], kc, vc, table, lens, 0.45, causal)
        assert np.array_equal(o[:, :, 0], o_d) and np.array_equal(lse[:, :, 0], lse_d)


def pin_fp8_decode_definition(orc):
    """E4M3 values the format fixes, and agreement with torch's float8_e4m3fn
    on all 256 codes (NaN codes included)."""
    import torch
    v = orc.fp8_e4m3_decode(np.array([0x00, 0x80, 0x38, 0xB8, 0x7E, 0xFE, 0x08, 0x07, 0x01, 0x40, 0x3C, 0x7F, 0xFF],
                                     dtype=np.uint8))
    exp = [0.0, -0.0, 1.0, -1.0, 448.0, -448.0, 2.0 ** -6, 7 * 2.0 ** -9, 2.0 ** -9, 2.0, 1.5]
    assert np.array_equal(v[:11], exp) and np.isnan(v[11]) and np.isnan(v[12])
    assert np.signbit(v[1]) and not np.signbit(v[0])
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    mine = orc.fp8_e4m3_decode(codes)
    assert np.array_equal(np.isnan(mine), np.isnan(ref))
    fin = ~np.isnan(ref)
    assert np.array_equal(mine[fin], ref[fin])
    # every finite code is distinct from its neighbours except the two zeros
    assert len(set(mine[fin].tolist())) == fin.sum() - 1


def pin_fp8_attention_descales(orc):
    """FP8 attention is the dense definition of the decoded tensors: scaling
    V's descale scales O; Q's or K's descale acts as the softmax scale."""
    rng = _rng(21)
    codes = lambda *sh: rng.integers(0, 256, size=sh).astype(np.uint8) & 0xF7  # no NaN codes (S.1111.111)
    q, k, v = codes(1, 2, 9, 8), codes(1, 1, 11, 8), codes(1, 1, 11, 8)
    for causal in (False, True):
        o, lse = orc.attention_fwd_fp8(q, k, v, 0.5, 0.25, 1.0, 0.3, causal)
        o2, lse2 = orc.attention_fwd_fp8(q, k, v, 0.5, 0.25, 2.0, 0.3, causal)
        assert np.array_equal(o2, 2.0 * o) and np.array_equal(lse2, lse)
        o3, lse3 = orc.attention_fwd_fp8(q, k, v, 1.0, 0.25, 1.0, 0.15, causal)
        assert np.abs(o3 - o).max() < 1e-13 and np.abs(lse3 - lse).max() < 1e-13
        dq, dk, dv = (orc.fp8_e4m3_decode(x) for x in (q, k, v))
        o4, lse4 = orc.attention_fwd(dq * 0.5, dk * 0.25, dv, 0.3, causal)
        assert np.array_equal(o4, o) and np.array_equal(lse4, lse)


# ---------------------------------------------------------------------------
# Large logits (max-stability checklist item)
# ---------------------------------------------------------------------------

def pin_large_logits_stable(orc):
    rng = _rng(17)
    d = 128
    q, k, v = _rand(rng, 1, 1, 64, d) * 8, _rand(rng, 1, 1, 64, d) * 8, _rand(rng, 1, 1, 64, d)
    scale = 1 / math.sqrt(d)
    o, lse = orc.attention_fwd(q, k, v, scale, True)
    assert np.isfinite(o).all() and np.isfinite(lse).all()
    s = scale * q[0, 0] @ k[0, 0].T
    assert np.abs(s).max() > 89.0  # exp overflows float32 beyond ~88.7
    # Negative control: the same row normalised without subtracting the max overflows in float32.
    with np.errstate(over="ignore", invalid="ignore"):
        naive = np.exp(s.astype(np.float32))
    assert not np.isfinite(naive).all()
    # Softmax is invariant to the max subtraction, so LSE - max lies in [0, ln Nk].
    m = np.where(np.tril(np.ones((64, 64), bool)), s, -np.inf).max(axis=1)
    gap = lse[0, 0] - m
    assert (gap >= -1e-12).all() and (gap <= math.log(64) + 1e-12).all()


def pin_packed_equal_lengths_equals_dense(orc):
    """A packed batch of equal-length sequences is the dense batch, flattened."""
    rng = _rng(31)
    b, hq, hkv, n, d = 3, 4, 2, 9, 4
    q, k, v, do = _rand(rng, b, hq, n, d), _rand(rng, b, hkv, n, d), _rand(rng, b, hkv, n, d), _rand(rng, b, hq, n, d)
    cu = np.arange(b + 1) * n
    for causal in (False, True):
        o, lse = orc.attention_fwd(q, k, v, 0.7, causal)
        op, lp = orc.attention_fwd_packed(q.reshape(-1, d), k.reshape(-1, d), v.reshape(-1, d), cu, cu, hq, hkv, 0.7,
                                          causal)
        assert np.abs(op - o.reshape(-1, d)).max() == 0 and np.abs(lp - lse.reshape(-1)).max() == 0
        g = orc.attention_bwd(q, k, v, do, 0.7, causal)
        gp = orc.attention_bwd_packed(q.reshape(-1, d), k.reshape(-1, d), v.reshape(-1, d), do.reshape(-1, d), cu, cu,
                                      hq, hkv, 0.7, causal)
        for a, c in zip(gp, g):
            assert np.abs(a - c.reshape(-1, d)).max() == 0


def pin_packed_mixed_lengths(orc):
    """Sequences of different query and key lengths (one empty), packed as
    [H, n_b, d] blocks one after another: every block of the result is the
    dense result of that sequence alone, and the other rows stay untouched."""
    rng = _rng(32)
    hq, hkv, d = 4, 2, 4
    lq, lk = [5, 0, 11, 3], [7, 4, 11, 1]
    seqs = [(_rand(rng, 1, hq, a, d), _rand(rng, 1, hkv, c, d), _rand(rng, 1, hkv, c, d), _rand(rng, 1, hq, a, d))
            for a, c in zip(lq, lk)]
    pack = lambda xs: np.concatenate([x[0].reshape(-1, d) for x in xs], axis=0)
    q, k, v, do = (pack([s_[i] for s_ in seqs]) for i in range(4))
    cu_q, cu_k = np.concatenate([[0], np.cumsum(lq)]), np.concatenate([[0], np.cumsum(lk)])
    for causal in (False, True):
        o, lse = orc.attention_fwd_packed(q, k, v, cu_q, cu_k, hq, hkv, 0.6, causal)
        dq, dk, dv = orc.attention_bwd_packed(q, k, v, do, cu_q, cu_k, hq, hkv, 0.6, causal)
        for bi, (qs, ks, vs, dos) in enumerate(seqs):
            rq, rk = slice(hq * cu_q[bi], hq * cu_q[bi + 1]), slice(hkv * cu_k[bi], hkv * cu_k[bi + 1])
            if lq[bi] == 0:
                assert o[rq].size == 0
                continue
            ob, lb = orc.attention_fwd(qs, ks, vs, 0.6, causal)
            # (rows that see no key carry LSE = -inf on both sides)
            assert np.array_equal(o[rq], ob.reshape(-1, d)) and np.array_equal(lse[rq], lb.reshape(-1))
            gb = orc.attention_bwd(qs, ks, vs, dos, 0.6, causal)
            assert np.array_equal(dq[rq], gb[0].reshape(-1, d))
            assert np.array_equal(dk[rk], gb[1].reshape(-1, d))
            assert np.array_equal(dv[rk], gb[2].reshape(-1, d))
        # the empty query sequence's keys get zero gradients
        rk1 = slice(hkv * cu_k[1], hkv * cu_k[2])
        assert np.abs(dk[rk1]).max() == 0 and np.abs(dv[rk1]).max() == 0


ALL_PINS = [
    pin_fp8_decode_definition,
    pin_fp8_attention_descales,
    pin_prefill_paged_equals_contiguous,
    pin_prefill_one_query_is_decode,
    pin_packed_equal_lengths_equals_dense,
    pin_packed_mixed_lengths,
    pin_worked_example_streaming,
    pin_worked_example_attention,
    pin_rows_sum_to_one,
    pin_constant_v,
    pin_key_permutation,
    pin_key_translation,
    pin_zero_query_closed_form,
    pin_single_key,
    pin_causal_first_row,
    pin_fully_masked_rows,
    pin_matches_torch_cpu_f64,
    pin_finite_differences,
    pin_backward_invariants,
    pin_gqa_equals_repeated_mha,
    pin_row_subset,
    pin_paged_decode_equals_contiguous,
    pin_paged_decode_table_permutation,
    pin_decode_empty_sequence,
    pin_large_logits_stable,
]
