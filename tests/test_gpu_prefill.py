"""GPU parity of the paged prefill (a chunk of queries over a paged KV cache)
against the float64 oracle."""

from __future__ import annotations

import pytest
import torch

from parity import assert_close, dev, f64, scale_for
from oracle import attention_f64 as orc
import synth_inputs as si

pytestmark = pytest.mark.gpu


def _fa():
    import exact_io_aware_47_amd as fa
    return fa


def run_prefill(q, kc, vc, table, lens, causal, scale=None):
    fa = _fa()
    o, lse = fa.prefill_paged(dev(q), dev(kc), dev(vc), dev(table), dev(lens), causal=causal, scale=scale)
    torch.cuda.synchronize()
    return o.cpu(), lse.cpu()


def check(q, kc, vc, table, lens, causal, dtype, scale=None):
    sc = scale_for(q.shape[-1]) if scale is None else scale
    o, lse = run_prefill(q, kc, vc, table, lens, causal, scale)
    ro, rl = orc.prefill_paged(f64(q), f64(kc), f64(vc), table.numpy(), lens.numpy(), sc, causal)
    assert_close("O", f64(o), ro, dtype, "o")
    assert_close("LSE", f64(lse), rl, dtype, "lse")


# B, Hq, Hkv, Nq, seq_lens, d, dtype, causal
CASES = [
    (2, 4, 2, 64, [300, 77], 128, "bf16", True),       # chunk shorter than the cache, ragged pages
    (1, 2, 2, 200, [200], 64, "f16", True),            # whole-sequence prefill
    (2, 2, 1, 100, [40, 257], 32, "bf16", True),       # chunk longer than one sequence: rows with no keys
    (2, 8, 2, 129, [1000, 513], 128, "bf16", False),
    (3, 3, 3, 17, [16, 33, 1], 64, "f16", False),
    (1, 2, 1, 70, [150], 32, "f32", True),
    (2, 2, 2, 33, [64, 90], 128, "f32", False),
    (1, 4, 4, 300, [1200], 64, "bf16", True),
    (2, 4, 1, 1, [500, 31], 128, "bf16", True),        # one query: the decode's case
    (2, 256, 64, 257, [300, 280], 64, "bf16", True),   # 8-wave work-groups (B * Hq * 2 tiles >= 512)
]


@pytest.mark.parametrize("B,Hq,Hkv,Nq,lens,d,dtype,causal", CASES,
                         ids=[f"B{c[0]}_H{c[1]}x{c[2]}_Nq{c[3]}_L{'-'.join(map(str, c[4]))}_d{c[5]}_{c[6]}_"
                              f"{'c' if c[7] else 'nc'}" for c in CASES])
def test_prefill_matches_oracle(B, Hq, Hkv, Nq, lens, d, dtype, causal):
    print(f"prefill case B={B} H={Hq}x{Hkv} Nq={Nq} lens={lens} d={d} {dtype} causal={causal}", flush=True)
    inputs = si.make_prefill_inputs(B, Hq, Hkv, Nq, lens, d, dtype, seed=6000 + Nq + sum(lens) + d, extra_blocks=5)
    check(*inputs, causal, dtype)


def test_prefill_clamps_out_of_range_lengths():
    """Lengths beyond the table row's reach (the last sequence included) are
    clamped to max_blocks * 16, negative ones to 0: compared with the oracle
    on the clamped lengths."""
    q, kc, vc, table, _ = si.make_prefill_inputs(3, 4, 2, 40, [100, 60, 90], 64, "bf16", seed=6101, extra_blocks=2)
    max_blocks = table.shape[1]
    for lens in ([100, -3, 2 ** 31 - 1], [5000, 60, 0]):
        given = torch.tensor(lens, dtype=torch.int32)
        clamped = given.clamp(0, max_blocks * 16)
        for causal in (True, False):
            o, lse = run_prefill(q, kc, vc, table, given, causal)
            ro, rl = orc.prefill_paged(f64(q), f64(kc), f64(vc), table.numpy(), clamped.numpy(), scale_for(64), causal)
            assert_close("O", f64(o), ro, "bf16", "o")
            assert_close("LSE", f64(lse), rl, "bf16", "lse")


def _scatter_into_pages(k, v, B, Hkv, N, d, seed):
    nb = -(-N // 16)
    perm = torch.randperm(B * nb + 3, generator=torch.Generator().manual_seed(seed))
    table = perm[: B * nb].view(B, nb).to(torch.int32)
    kc = torch.zeros(B * nb + 3, Hkv, 16, d, dtype=k.dtype)
    vc = torch.zeros_like(kc)
    for b in range(B):
        for t in range(N):
            kc[table[b, t // 16], :, t % 16] = k[b, :, t]
            vc[table[b, t // 16], :, t % 16] = v[b, :, t]
    return kc, vc, table


def test_prefill_equals_dense_forward_bitwise():
    """Keys scattered into pages by host code: on a grid that runs the 8-wave
    kernel for both (B * Hq * ceil(N / 256) >= 512), the paged call gives
    bitwise the dense forward's O and LSE (same tiles, same arithmetic
    order)."""
    fa = _fa()
    B, Hq, Hkv, N, d = 2, 128, 64, 333, 128
    assert B * Hq * -(-N // 256) >= 512
    q, k, v, _ = si.make_attention_inputs(B, Hq, Hkv, N, N, d, "bf16", seed=93)
    kc, vc, table = _scatter_into_pages(k, v, B, Hkv, N, d, 94)
    lens = torch.full((B,), N, dtype=torch.int32)
    for causal in (True, False):
        o, lse = fa.fwd(dev(q), dev(k), dev(v), causal=causal)
        po, pl = fa.prefill_paged(dev(q), dev(kc), dev(vc), dev(table), dev(lens), causal=causal)
        torch.cuda.synchronize()
        assert torch.equal(o, po) and torch.equal(lse, pl)


@pytest.mark.parametrize("d", [64, 128])
def test_prefill_and_dense_forward_on_a_short_grid(d):
    """A short grid (a key-split kernel for both: at d=64 the causal call runs
    the 4-wave one): the paged call gives bitwise the dense forward's O and
    LSE, and both match the oracle."""
    fa = _fa()
    B, Hq, Hkv, N = 2, 4, 2, 333
    q, k, v, _ = si.make_attention_inputs(B, Hq, Hkv, N, N, d, "bf16", seed=93)
    kc, vc, table = _scatter_into_pages(k, v, B, Hkv, N, d, 94)
    lens = torch.full((B,), N, dtype=torch.int32)
    for causal in (True, False):
        o, lse = fa.fwd(dev(q), dev(k), dev(v), causal=causal)
        po, pl = fa.prefill_paged(dev(q), dev(kc), dev(vc), dev(table), dev(lens), causal=causal)
        torch.cuda.synchronize()
        assert torch.equal(o, po) and torch.equal(lse, pl)
        ro, rl = orc.attention_fwd(f64(q), f64(k), f64(v), scale_for(d), causal)
        assert_close("O", f64(o.cpu()), ro, "bf16", "o")
        assert_close("LSE", f64(lse.cpu()), rl, "bf16", "lse")


def test_prefill_bad_table_entry_reads_zero_page():
    """A table entry outside [0, num_blocks) is read as a page of zeros (no fault)."""
    B, Hq, Hkv, Nq, d = 1, 2, 2, 40, 64
    q, kc, vc, table, lens = si.make_prefill_inputs(B, Hq, Hkv, Nq, [48], d, "bf16", seed=95)
    bad = table.clone()
    bad[0, 1] = 1 << 20
    o, lse = run_prefill(q, kc, vc, bad, lens, True)
    kz, vz = kc.clone(), vc.clone()
    kz[table[0, 1]] = 0
    vz[table[0, 1]] = 0
    ro, rl = orc.prefill_paged(f64(q), f64(kz), f64(vz), table.numpy(), lens.numpy(), scale_for(d), True)
    assert_close("O", f64(o), ro, "bf16", "o")
    assert_close("LSE", f64(lse), rl, "bf16", "lse")


def test_prefill_workload_prefill_paged_bf16():
    """The chunked-prefill workload at full size, checked on sampled heads."""
    w = si.WORKLOADS["prefill_paged_bf16"]
    q, kc, vc, table, lens = si.workload_prefill_inputs(w)
    o, lse = run_prefill(q, kc, vc, table, lens, w.causal)
    for b, h in ((0, 0), (1, 13), (3, 31)):
        sl = (slice(b, b + 1), slice(h, h + 1))
        hkv = h // (w.Hq // w.Hkv)
        ro, rl = orc.prefill_paged(f64(q[sl]), f64(kc[:, hkv:hkv + 1]), f64(vc[:, hkv:hkv + 1]),
                                   table[b:b + 1].numpy(), lens[b:b + 1].numpy(), w.scale, w.causal)
        assert_close(f"O[{b},{h}]", f64(o[sl]), ro, w.dtype, "o")
        assert_close(f"LSE[{b},{h}]", f64(lse[sl]), rl, w.dtype, "lse")
