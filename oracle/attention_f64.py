"""Float64 CPU oracle for exact attention: plain, slow, obviously correct.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this module.  The GPU library never calls it, and
this module imports nothing from the GPU library.

What is computed follows the pages' own statement of the problem:

* "FlashAttention and efficient attention kernels" (plumephp tutorial),
  section "Standard attention" (three steps S = Q Kᵀ, P = softmax(S), O = P V)
  and the concept page "Flash-Attention" (awesome-system-papers), section
  "Core idea", which writes the scaled form softmax(Q Kᵀ/√d) V and states that
  the tiled method is mathematically equal to it.  The oracle is therefore the
  three-step definition itself, in float64, one (batch, head) at a time.
* Backward: the tutorial's sections "Backward" and "Backward recompute flow"
  say only that dQ/dK/dV are obtained from Q, K, V, the saved statistics and
  dO.  The pages print no gradient formula, so the oracle uses the plain chain
  rule of the three-step definition (pinned by finite differences and by
  torch's CPU float64 autograd in the tests).
* Streaming normaliser: the tutorial's sections "Online softmax",
  "Correction formula" and the worked example ("streaming process"), and the
  related-work page's paper #1 (Online normalizer calculation for softmax).
* Decode over a paged KV cache: the tutorial's "Variant family" section
  (FlashDecoding splits the KV sequence; PagedAttention reads non-contiguous
  fixed-size blocks) and the related-work page's paper #5 (PagedAttention).
  The oracle gathers the pages back into a contiguous sequence and applies the
  three-step definition with one query row.

Readings where the pages are silent (each listed with its reason in the
design notes):
* scale is an explicit argument applied to S before the mask and the max;
* causal masking is bottom-right aligned: key j is visible to query i iff
  j <= i + (Nk - Nq);
* a row with no visible key has O = 0, LSE = -inf and zero gradients;
* grouped-query heads are contiguous groups: kv head = q head // (Hq / Hkv);
* LSE = m + ln(l) in natural log;
* KV cache pages are laid out [num_blocks, Hkv, block_size, d];
* a packed (variable-length) batch stores sequence b's rows of every head as
  one [H, n_b, d] block starting at row H * cu[b]; each sequence is attended
  on its own.
* Paged prefill: the concept page's key observation 4 and the tutorial's
  "Variant family" section (PagedAttention fused with the tiled kernel).  A
  chunk of Nq new queries per sequence attends to that sequence's cached
  tokens; the queries are the sequence's last Nq positions, so the causal
  mask is the same bottom-right alignment as the dense definition.
* FP8 forward: the concept page's key observations (FlashAttention-3's FP8
  path) and the tutorial's validation checklist (FP8).  The pages give no
  encoding or scaling recipe.  Reading: inputs are OCP FP8 E4M3 codes (sign,
  4 exponent bits with bias 7, 3 mantissa bits; exponent field 0 is
  subnormal; S.1111.111 is NaN; no infinities) times one float32 descale
  factor per tensor.  The oracle decodes the codes from that definition and
  applies the dense definition to the decoded values.
* Packed batches: the related-work page's repository comparison (varlen
  support in the reference implementation), the concept page's key
  observation 4 (variable-length packing) and the tutorial's validation
  checklist (variable-length sequences).  The pages give no layout; the
  oracle splits the packed arrays into sequences and applies the dense
  definition to each.

Every function here is pinned in ``tests/test_oracle.py`` against values and
properties that the pages and the mathematics fix.
"""

from __future__ import annotations

import math

import numpy as np

__all__ = [
    "visible_mask",
    "attention_probs",
    "attention_fwd",
    "attention_bwd",
    "decode_paged",
    "prefill_paged",
    "fp8_e4m3_decode",
    "attention_fwd_fp8",
    "attention_fwd_packed",
    "attention_bwd_packed",
    "gather_pages",
    "online_softmax_stats",
    "merge_softmax_stats",
]


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def visible_mask(nq: int, nk: int, causal: bool, row_ids=None, nq_total=None) -> np.ndarray:
    """Boolean [nq, nk] mask of the (query, key) pairs that take part.

    Causal alignment is bottom-right: query row i of a query sequence of
    length ``nq_total`` sees key j iff ``j <= i + (nk - nq_total)``.  To
    evaluate a subset of rows of a longer query sequence, pass their indices
    in ``row_ids`` and the full length in ``nq_total`` (defaults: all rows,
    ``nq_total = nq``).
    """
    if not causal:
        return np.ones((nq, nk), dtype=bool)
    rows = np.arange(nq) if row_ids is None else np.asarray(row_ids, dtype=np.int64)
    total = nq if nq_total is None else int(nq_total)
    return np.arange(nk)[None, :] <= (rows + (nk - total))[:, None]


def attention_probs(q, k, scale: float, causal: bool, row_ids=None, nq_total=None):
    """P = softmax(scale * q kᵀ) row-wise, with masked entries exactly 0.

    q: [Nq, d], k: [Nk, d].  Returns (P [Nq, Nk], LSE [Nq]).  A row with no
    visible key returns P = 0 and LSE = -inf.  ``row_ids``/``nq_total`` select
    the causal horizon of a subset of rows (see ``visible_mask``).
    """
    q = _f64(q)
    k = _f64(k)
    s = scale * (q @ k.T)
    vis = visible_mask(q.shape[0], k.shape[0], causal, row_ids, nq_total)
    s = np.where(vis, s, -np.inf)
    m = s.max(axis=1) if s.shape[1] > 0 else np.full(s.shape[0], -np.inf)
    empty = ~np.isfinite(m)
    m_safe = np.where(empty, 0.0, m)
    e = np.exp(s - m_safe[:, None])  # exp(-inf) = 0 on masked entries
    l = e.sum(axis=1)
    p = np.where(empty[:, None], 0.0, e / np.where(empty, 1.0, l)[:, None])
    lse = np.where(empty, -np.inf, m_safe + np.log(np.where(empty, 1.0, l)))
    return p, lse


def _check_heads(hq: int, hkv: int) -> int:
    if hkv <= 0 or hq % hkv != 0:
        raise ValueError(f"Hq={hq} must be a positive multiple of Hkv={hkv}")
    return hq // hkv


def attention_fwd(q, k, v, scale: float, causal: bool, row_ids=None, nq_total=None):
    """Exact attention forward.

    q: [B, Hq, Nq, d]; k, v: [B, Hkv, Nk, d].  Returns O [B, Hq, Nq, d] and
    LSE [B, Hq, Nq] in float64.  Query head h reads kv head h // (Hq/Hkv).
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    bsz, hq, nq, d = q.shape
    hkv = k.shape[1]
    g = _check_heads(hq, hkv)
    o = np.zeros((bsz, hq, nq, v.shape[3]))
    lse = np.zeros((bsz, hq, nq))
    for b in range(bsz):
        for h in range(hq):
            p, lse[b, h] = attention_probs(q[b, h], k[b, h // g], scale, causal, row_ids, nq_total)
            o[b, h] = p @ v[b, h // g]
    return o, lse


def attention_bwd(q, k, v, do, scale: float, causal: bool, row_ids=None, nq_total=None):
    """Gradients of sum(O * dO) with respect to Q, K and V.

    Plain chain rule through the three-step definition:
        O  = P V,  P = softmax(S) row-wise,  S = scale * Q Kᵀ (masked)
        dV = Pᵀ dO
        dP = dO Vᵀ
        dS = P ∘ (dP − D 1ᵀ),  D_i = Σ_c dO_ic O_ic   (= Σ_j P_ij dP_ij)
        dQ = scale · dS K,      dK = scale · dSᵀ Q
    For grouped heads, dK and dV of a kv head are summed over its query heads.
    Returns (dQ, dK, dV) in float64 with the shapes of q, k, v.
    """
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    bsz, hq, nq, d = q.shape
    hkv = k.shape[1]
    g = _check_heads(hq, hkv)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for b in range(bsz):
        for h in range(hq):
            kh, vh = k[b, h // g], v[b, h // g]
            p, _ = attention_probs(q[b, h], kh, scale, causal, row_ids, nq_total)
            o = p @ vh
            dd = (do[b, h] * o).sum(axis=1)
            dp = do[b, h] @ vh.T
            ds = p * (dp - dd[:, None])
            dq[b, h] = scale * (ds @ kh)
            dk[b, h // g] += scale * (ds.T @ q[b, h])
            dv[b, h // g] += p.T @ do[b, h]
    return dq, dk, dv


def fp8_e4m3_decode(codes) -> np.ndarray:
    """Values of OCP FP8 E4M3 codes (uint8 array) in float64.

    Bit 7 is the sign, bits 6..3 the exponent e (bias 7), bits 2..0 the
    mantissa f: e > 0 gives (1 + f/8) * 2^(e-7), e = 0 gives (f/8) * 2^-6,
    and e = 15 with f = 7 is NaN (the format has no infinities).
    """
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    f = (c & 0x7).astype(np.float64)
    mag = np.where(e > 0, (1.0 + f / 8.0) * np.exp2(e - 7.0), (f / 8.0) * 2.0 ** -6)
    mag = np.where((e == 15) & (f == 7), np.nan, mag)
    return sign * mag


def attention_fwd_fp8(q_codes, k_codes, v_codes, q_descale: float, k_descale: float, v_descale: float,
                      scale: float, causal: bool):
    """Forward on FP8 inputs: each tensor is its E4M3 codes times its descale.
    q_codes [B, Hq, Nq, d], k_codes / v_codes [B, Hkv, Nk, d] (uint8).
    Returns O [B, Hq, Nq, d], LSE [B, Hq, Nq] of the decoded tensors."""
    q = fp8_e4m3_decode(q_codes) * q_descale
    k = fp8_e4m3_decode(k_codes) * k_descale
    v = fp8_e4m3_decode(v_codes) * v_descale
    return attention_fwd(q, k, v, scale, causal)


def _unpack(x, cu, h: int, b: int):
    """Sequence b of a packed [sum_b h*n_b, d] array as [1, h, n_b, d]."""
    n = int(cu[b + 1]) - int(cu[b])
    r0 = h * int(cu[b])
    return x[r0:r0 + h * n].reshape(1, h, n, x.shape[-1])


def attention_fwd_packed(q, k, v, cu_q, cu_k, hq: int, hkv: int, scale: float, causal: bool):
    """Forward of a packed batch: each sequence through attention_fwd.
    Returns O like q and LSE [sum_b hq*n_b] (float64)."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    o = np.zeros_like(q)
    lse = np.zeros(q.shape[0])
    for b in range(len(cu_q) - 1):
        nq = int(cu_q[b + 1]) - int(cu_q[b])
        if nq == 0:
            continue
        ob, lb = attention_fwd(_unpack(q, cu_q, hq, b), _unpack(k, cu_k, hkv, b), _unpack(v, cu_k, hkv, b),
                               scale, causal)
        r0 = hq * int(cu_q[b])
        o[r0:r0 + hq * nq] = ob.reshape(hq * nq, -1)
        lse[r0:r0 + hq * nq] = lb.reshape(-1)
    return o, lse


def attention_bwd_packed(q, k, v, do, cu_q, cu_k, hq: int, hkv: int, scale: float, causal: bool):
    """Backward of a packed batch: each sequence through attention_bwd.
    Returns dQ, dK, dV with the packed shapes of q, k, v (float64)."""
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    for b in range(len(cu_q) - 1):
        nq = int(cu_q[b + 1]) - int(cu_q[b])
        nk = int(cu_k[b + 1]) - int(cu_k[b])
        if nq == 0 or nk == 0:
            continue
        gq, gk, gv = attention_bwd(_unpack(q, cu_q, hq, b), _unpack(k, cu_k, hkv, b), _unpack(v, cu_k, hkv, b),
                                   _unpack(do, cu_q, hq, b), scale, causal)
        rq, rk = hq * int(cu_q[b]), hkv * int(cu_k[b])
        dq[rq:rq + hq * nq] = gq.reshape(hq * nq, -1)
        dk[rk:rk + hkv * nk] = gk.reshape(hkv * nk, -1)
        dv[rk:rk + hkv * nk] = gv.reshape(hkv * nk, -1)
    return dq, dk, dv


def gather_pages(cache, block_table_row, seq_len: int) -> np.ndarray:
    """Contiguous [Hkv, seq_len, d] keys (or values) of one sequence.

    cache: [num_blocks, Hkv, block_size, d]; token t lives in page
    ``block_table_row[t // block_size]`` at slot ``t % block_size``.
    """
    cache = np.asarray(cache)
    num_blocks, hkv, bs, d = cache.shape
    out = np.zeros((hkv, seq_len, d), dtype=np.float64)
    for t in range(0, seq_len, bs):
        page = int(block_table_row[t // bs])
        if not 0 <= page < num_blocks:
            raise IndexError(f"block table entry {page} outside [0, {num_blocks})")
        n = min(bs, seq_len - t)
        out[:, t:t + n, :] = cache[page, :, :n, :]
    return out


def decode_paged(q, k_cache, v_cache, block_table, seq_lens, scale: float):
    """One-token decode over a paged KV cache.

    q: [B, Hq, d]; k_cache, v_cache: [num_blocks, Hkv, block_size, d];
    block_table: [B, max_blocks] integer page ids; seq_lens: [B] token counts.
    The single query row sees every cached token of its sequence (it is the
    last position), so no mask applies.  Returns O [B, Hq, d], LSE [B, Hq];
    a sequence of length 0 gives O = 0 and LSE = -inf.
    """
    q = _f64(q)
    bsz, hq, d = q.shape
    hkv = np.asarray(k_cache).shape[1]
    g = _check_heads(hq, hkv)
    o = np.zeros((bsz, hq, d))
    lse = np.zeros((bsz, hq))
    for b in range(bsz):
        n = int(seq_lens[b])
        kb = gather_pages(k_cache, block_table[b], n)
        vb = gather_pages(v_cache, block_table[b], n)
        for h in range(hq):
            p, lse_row = attention_probs(q[b, h][None, :], kb[h // g], scale, False)
            o[b, h] = (p @ vb[h // g])[0]
            lse[b, h] = lse_row[0]
    return o, lse


def prefill_paged(q, k_cache, v_cache, block_table, seq_lens, scale: float, causal: bool):
    """Attention of a chunk of queries over a paged KV cache.

    q: [B, Hq, Nq, d], the last Nq positions of each sequence;
    k_cache, v_cache: [num_blocks, Hkv, block_size, d]; block_table:
    [B, max_blocks]; seq_lens: [B] cached tokens per sequence (the chunk's
    own tokens included).  Each sequence's keys are gathered back into a
    contiguous [Hkv, seq_len, d] block and the dense definition applies,
    with the bottom-right causal alignment (query i of the chunk sees key j
    iff j <= i + seq_len - Nq).  Returns O [B, Hq, Nq, d], LSE [B, Hq, Nq].
    """
    q = _f64(q)
    bsz, hq, nq, d = q.shape
    o = np.zeros((bsz, hq, nq, d))
    lse = np.zeros((bsz, hq, nq))
    for b in range(bsz):
        n = int(seq_lens[b])
        kb = gather_pages(k_cache, block_table[b], n)[None]
        vb = gather_pages(v_cache, block_table[b], n)[None]
        o[b], lse[b] = (x[0] for x in attention_fwd(q[b][None], kb, vb, scale, causal))
    return o, lse


def online_softmax_stats(x, block: int):
    """Streaming (max, sum) of one row, visiting it ``block`` entries at a time.

    This is the update of the tutorial's "Online softmax" and "Correction
    formula" sections: on each new block the running max becomes
    max(old max, block max), the old running sum is rescaled by
    exp(old max − new max), and the block's exponentials, taken relative to the
    new max, are added.  Returns (m, l) with softmax denominator
    l = Σ exp(x − m).  An empty or all −inf row gives (−inf, 0).
    """
    x = _f64(x).ravel()
    m, l = -math.inf, 0.0
    for start in range(0, x.size, block):
        blk = x[start:start + block]
        m_new = max(m, float(blk.max()))
        if m_new == -math.inf:
            continue
        rescale = 0.0 if m == -math.inf else math.exp(m - m_new)
        l = l * rescale + float(np.exp(blk - m_new).sum())
        m = m_new
    return m, l


def merge_softmax_stats(m_a: float, l_a: float, m_b: float, l_b: float):
    """Combine two partial (max, sum) pairs taken over disjoint parts of a row.

    Each part's sum is relative to its own max, so both are rescaled to the
    common max:  M = max(m_a, m_b),  L = l_a·exp(m_a − M) + l_b·exp(m_b − M).
    (When part b's max is already the common max this is the tutorial's
    correction formula verbatim.)  Empty parts are (−inf, 0).
    """
    mx = max(m_a, m_b)
    if mx == -math.inf:
        return -math.inf, 0.0
    wa = 0.0 if m_a == -math.inf else math.exp(m_a - mx)
    wb = 0.0 if m_b == -math.inf else math.exp(m_b - mx)
    return mx, l_a * wa + l_b * wb
