"""Seeded synthetic inputs for the attention workloads.

This module only draws random numbers and casts them; it holds none of the
attention arithmetic.  Both the GPU-side tests/benchmark and the float64
oracle consume exactly the tensors produced here, so the oracle sees the very
values the kernels see (the cast to the compute dtype is round-to-nearest-even
and happens once, here; the oracle upcasts the already-rounded values).

Workloads (shapes, dtypes and value distributions of the five attention
configurations; the pages themselves publish no inputs or seeds):

* ``mha_f32_small``   B=1  H=1  N=128    d=32  fp32, non-causal
* ``mha_f16``         B=4  H=8  N=1024   d=64  fp16, causal and non-causal
* ``mha_bf16_4k``     B=2  H=16 N=4096   d=128 bf16, causal (training/prefill)
* ``mha_bf16_16k``    B=1  H=16 N=16384  d=128 bf16, causal, Q and K times 8
* ``decode_gqa_paged`` B=8 Hq=32 Hkv=8 Nk=32768 d=128 bf16, 16-token pages
  reached through a seeded random permutation block table.
* ``gqa_bf16_4k``     B=2 Hq=32 Hkv=8 N=4096 d=128 bf16, causal (grouped-query
  training shape; not one of the five configurations)
* ``prefill_paged_bf16`` B=4 Hq=32 Hkv=8 d=128 bf16, causal: a chunk of 1024
  new queries per sequence over 8192 cached tokens in 16-token pages reached
  through a seeded random permutation block table (chunked prefill; not one
  of the five configurations)
* ``mha_fp8_4k``      B=2 H=16 N=4096 d=128, causal, FP8 E4M3 inputs: the
  N(0,1) draws of Q, K, V divided by a per-tensor descale amax/448 and
  rounded to E4M3 (the FP8 forward; not one of the five configurations)
* ``varlen_bf16``     a packed batch of 16 causal sequences (Hq=Hkv=16,
  d=128, bf16) whose lengths are drawn uniformly from [1, 4096] by the seeded
  generator (not one of the five configurations; the pages name packed
  variable-length batches but give no length mix)

Draw order for a forward/backward workload: Q, K, V, dO, each i.i.d. N(0, 1)
from ``torch.Generator('cpu').manual_seed(seed)``.  For decode: Q, K cache,
V cache, then the page permutation (paged prefill: the same, with Nq query
rows per sequence).  For a packed batch: the sequence lengths
(when drawn), then Q, K, V, dO.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch

__all__ = [
    "AttnWorkload",
    "DecodeWorkload",
    "WORKLOADS",
    "DTYPES",
    "make_attention_inputs",
    "make_decode_inputs",
    "make_packed_inputs",
    "make_prefill_inputs",
    "make_fp8_inputs",
    "PrefillWorkload",
    "PackedWorkload",
]

DTYPES = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


@dataclass(frozen=True)
class AttnWorkload:
    name: str
    B: int
    Hq: int
    Hkv: int
    Nq: int
    Nk: int
    d: int
    dtype: str
    causal: tuple
    seed: int
    qk_mult: float = 1.0

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)


@dataclass(frozen=True)
class DecodeWorkload:
    name: str
    B: int
    Hq: int
    Hkv: int
    seq_len: int
    d: int
    dtype: str
    seed: int
    block_size: int = 16
    extra_blocks: int = 0  # unused pages in the cache beyond what sequences need

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    @property
    def max_blocks(self) -> int:
        return -(-self.seq_len // self.block_size)

    @property
    def num_blocks(self) -> int:
        return self.B * self.max_blocks + self.extra_blocks


@dataclass(frozen=True)
class PrefillWorkload:
    name: str
    B: int
    Hq: int
    Hkv: int
    Nq: int           # new queries per sequence (the chunk)
    seq_len: int      # cached tokens per sequence, the chunk included
    d: int
    dtype: str
    causal: bool
    seed: int
    block_size: int = 16

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)


@dataclass(frozen=True)
class PackedWorkload:
    name: str
    B: int            # sequences in the batch
    Hq: int
    Hkv: int
    max_len: int      # lengths drawn uniformly from [1, max_len]
    d: int
    dtype: str
    causal: bool
    seed: int

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)


WORKLOADS = {
    "mha_f32_small": AttnWorkload("mha_f32_small", 1, 1, 1, 128, 128, 32, "f32", (False,), 47001),
    "mha_f16": AttnWorkload("mha_f16", 4, 8, 8, 1024, 1024, 64, "f16", (True, False), 47002),
    "mha_bf16_4k": AttnWorkload("mha_bf16_4k", 2, 16, 16, 4096, 4096, 128, "bf16", (True,), 47003),
    "mha_bf16_16k": AttnWorkload("mha_bf16_16k", 1, 16, 16, 16384, 16384, 128, "bf16", (True,), 47004,
                                 qk_mult=8.0),
    "decode_gqa_paged": DecodeWorkload("decode_gqa_paged", 8, 32, 8, 32768, 128, "bf16", 47005),
    # grouped-query training shape: four query heads per K/V head
    "gqa_bf16_4k": AttnWorkload("gqa_bf16_4k", 2, 32, 8, 4096, 4096, 128, "bf16", (True,), 47006),
    # FP8 forward on the training shape (E4M3 codes with amax/448 descales)
    "mha_fp8_4k": AttnWorkload("mha_fp8_4k", 2, 16, 16, 4096, 4096, 128, "fp8", (True,), 47009),
    # chunked prefill over a paged cache
    "prefill_paged_bf16": PrefillWorkload("prefill_paged_bf16", 4, 32, 8, 1024, 8192, 128, "bf16", True, 47008),
    # packed batch of variable-length causal sequences
    "varlen_bf16": PackedWorkload("varlen_bf16", 16, 16, 16, 4096, 128, "bf16", True, 47007),
}


def _normal(gen: torch.Generator, shape, mult: float = 1.0) -> torch.Tensor:
    x = torch.randn(*shape, generator=gen, dtype=torch.float32)
    if mult != 1.0:
        x.mul_(mult)  # a power of two: exact in every binary format
    return x


def make_attention_inputs(B, Hq, Hkv, Nq, Nk, d, dtype: str, seed: int, qk_mult: float = 1.0):
    """Q [B,Hq,Nq,d], K/V [B,Hkv,Nk,d], dO [B,Hq,Nq,d] on the CPU in ``dtype``.

    Drawn in the order Q, K, V, dO from one seeded CPU generator as float32
    N(0,1) (Q and K multiplied by ``qk_mult``), then rounded to ``dtype``.
    """
    tdt = DTYPES[dtype]
    gen = torch.Generator(device="cpu").manual_seed(int(seed))
    q = _normal(gen, (B, Hq, Nq, d), qk_mult).to(tdt)
    k = _normal(gen, (B, Hkv, Nk, d), qk_mult).to(tdt)
    v = _normal(gen, (B, Hkv, Nk, d)).to(tdt)
    do = _normal(gen, (B, Hq, Nq, d)).to(tdt)
    return q, k, v, do


def make_decode_inputs(B, Hq, Hkv, seq_lens, d, dtype: str, seed: int, block_size: int = 16,
                       extra_blocks: int = 0):
    """Inputs of a paged decode step.

    Returns (q [B,Hq,d], k_cache, v_cache [num_blocks,Hkv,block_size,d],
    block_table [B,max_blocks] int32, seq_lens [B] int32).  ``seq_lens`` is an
    int (same length for every sequence) or a list.  Every sequence gets
    ``max_blocks`` table entries; the pages are a seeded random permutation of
    all ``num_blocks`` cache pages, so the table is a bijection onto the used
    pages and neighbouring tokens of a sequence live in unrelated pages.
    """
    tdt = DTYPES[dtype]
    if isinstance(seq_lens, int):
        seq_lens = [seq_lens] * B
    seq_lens = torch.tensor(seq_lens, dtype=torch.int32)
    max_blocks = max(1, -(-int(seq_lens.max()) // block_size))
    num_blocks = B * max_blocks + extra_blocks
    gen = torch.Generator(device="cpu").manual_seed(int(seed))
    q = _normal(gen, (B, Hq, d)).to(tdt)
    k_cache = _normal(gen, (num_blocks, Hkv, block_size, d)).to(tdt)
    v_cache = _normal(gen, (num_blocks, Hkv, block_size, d)).to(tdt)
    perm = torch.randperm(num_blocks, generator=gen)
    block_table = perm[: B * max_blocks].view(B, max_blocks).to(torch.int32).contiguous()
    return q, k_cache, v_cache, block_table, seq_lens


def make_fp8_inputs(B, Hq, Hkv, Nq, Nk, d, seed: int):
    """FP8 inputs: float32 N(0,1) draws of Q, K, V (in that order), each
    divided by its per-tensor descale amax / 448 and rounded to E4M3
    (torch.float8_e4m3fn, round to nearest even).  Returns (q, k, v codes,
    (q_descale, k_descale, v_descale)); the value of an element is its code
    times its tensor's descale."""
    gen = torch.Generator(device="cpu").manual_seed(int(seed))
    xs = [_normal(gen, (B, Hq, Nq, d)), _normal(gen, (B, Hkv, Nk, d)), _normal(gen, (B, Hkv, Nk, d))]
    out, desc = [], []
    for x in xs:
        ds = float(x.abs().max()) / 448.0
        out.append((x / ds).to(torch.float8_e4m3fn))
        desc.append(ds)
    return out[0], out[1], out[2], tuple(desc)


def make_prefill_inputs(B, Hq, Hkv, Nq, seq_lens, d, dtype: str, seed: int, block_size: int = 16,
                        extra_blocks: int = 0):
    """Inputs of a chunked prefill over a paged cache: as make_decode_inputs,
    but with Nq query rows per sequence (q [B, Hq, Nq, d]).  Draw order: Q,
    K cache, V cache, page permutation."""
    tdt = DTYPES[dtype]
    if isinstance(seq_lens, int):
        seq_lens = [seq_lens] * B
    seq_lens = torch.tensor(seq_lens, dtype=torch.int32)
    max_blocks = max(1, -(-int(seq_lens.max()) // block_size))
    num_blocks = B * max_blocks + extra_blocks
    gen = torch.Generator(device="cpu").manual_seed(int(seed))
    q = _normal(gen, (B, Hq, Nq, d)).to(tdt)
    k_cache = _normal(gen, (num_blocks, Hkv, block_size, d)).to(tdt)
    v_cache = _normal(gen, (num_blocks, Hkv, block_size, d)).to(tdt)
    perm = torch.randperm(num_blocks, generator=gen)
    block_table = perm[: B * max_blocks].view(B, max_blocks).to(torch.int32).contiguous()
    return q, k_cache, v_cache, block_table, seq_lens


def workload_prefill_inputs(w: PrefillWorkload):
    return make_prefill_inputs(w.B, w.Hq, w.Hkv, w.Nq, w.seq_len, w.d, w.dtype, w.seed, w.block_size)


def make_packed_inputs(lens_q, lens_k, Hq, Hkv, d, dtype: str, seed: int, max_len: int = 0):
    """Inputs of a packed (variable-length) batch.

    ``lens_q`` / ``lens_k`` list the query / key count of each sequence; with
    ``lens_q=None`` and ``max_len > 0``, ``lens_k`` must be the number of
    sequences and equal query and key lengths are drawn uniformly from
    [1, max_len] (first, from the same generator).  Returns
    (q [Hq*total_q, d], k, v [Hkv*total_k, d], dO like q, cu_q, cu_k [B+1]
    int32), where head h of sequence b occupies rows H*cu[b] + h*n_b, ...
    (each sequence's dense [H, n_b, d] block, concatenated).
    """
    tdt = DTYPES[dtype]
    gen = torch.Generator(device="cpu").manual_seed(int(seed))
    if lens_q is None:
        lens_q = torch.randint(1, max_len + 1, (int(lens_k),), generator=gen).tolist()
        lens_k = list(lens_q)
    if len(lens_q) != len(lens_k):
        raise ValueError("lens_q and lens_k must have one entry per sequence")
    cu_q = torch.tensor([0] + list(lens_q), dtype=torch.int64).cumsum(0).to(torch.int32)
    cu_k = torch.tensor([0] + list(lens_k), dtype=torch.int64).cumsum(0).to(torch.int32)
    tq, tk = int(cu_q[-1]), int(cu_k[-1])
    q = _normal(gen, (Hq * tq, d)).to(tdt)
    k = _normal(gen, (Hkv * tk, d)).to(tdt)
    v = _normal(gen, (Hkv * tk, d)).to(tdt)
    do = _normal(gen, (Hq * tq, d)).to(tdt)
    return q, k, v, do, cu_q, cu_k


def workload_packed_inputs(w: PackedWorkload):
    return make_packed_inputs(None, w.B, w.Hq, w.Hkv, w.d, w.dtype, w.seed, max_len=w.max_len)


def workload_attention_inputs(w: AttnWorkload):
    return make_attention_inputs(w.B, w.Hq, w.Hkv, w.Nq, w.Nk, w.d, w.dtype, w.seed, w.qk_mult)


def workload_decode_inputs(w: DecodeWorkload):
    return make_decode_inputs(w.B, w.Hq, w.Hkv, w.seq_len, w.d, w.dtype, w.seed, w.block_size,
                              w.extra_blocks)
