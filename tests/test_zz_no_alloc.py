"""GPU test of the allocation-free decode (flash_attn_decode_paged_noalloc):
through the C ABI, its output equals flash_attn_decode_paged's (same kernels,
same split count) on two calls in a row, the second with a smaller input,
and is within the 16-bit tolerances of the float64 oracle."""

from __future__ import annotations

import math

import pytest
import torch

from parity import assert_close, dev, f64
from oracle import attention_f64 as orc
import synth_inputs as si

pytestmark = pytest.mark.gpu


def _case(B, Hq, Hkv, lens, d, dtype, splits, seed):
    import exact_io_aware_47_amd as fa
    print(f"noalloc decode B={B} H={Hq}x{Hkv} lens={lens} d={d} {dtype} splits={splits}", flush=True)
    q, kc, vc, table, sl = si.make_decode_inputs(B, Hq, Hkv, lens, d, dtype, seed=seed, extra_blocks=3)
    qd, kcd, vcd, td, sld = dev(q), dev(kc), dev(vc), dev(table), dev(sl)
    sc = 1.0 / math.sqrt(d)
    o_ref, l_ref = fa.decode_paged(qd, kcd, vcd, td, sld, scale=sc, num_splits=splits)
    out = torch.full_like(qd, float("nan"))
    lse = torch.full((B, Hq), float("nan"), dtype=torch.float32, device="cuda")
    o, l = fa.decode_paged_noalloc(qd, kcd, vcd, td, sld, scale=sc, num_splits=splits, out=out, lse=lse)
    torch.cuda.synchronize()
    assert o.data_ptr() == out.data_ptr() and l.data_ptr() == lse.data_ptr()
    assert torch.equal(o, o_ref) and torch.equal(l, l_ref)
    ro, rl = orc.decode_paged(f64(q), kc.float().numpy(), vc.float().numpy(), table.numpy(), sl.numpy(), sc)
    assert_close("O", f64(o.cpu()), ro, dtype, "o")
    assert_close("LSE", f64(l.cpu()), rl, dtype, "lse")


def test_noalloc_decode_matches_decode_paged_twice():
    # First call: grouped heads, ragged lengths, the automatic split count.
    _case(4, 32, 8, [5000, 17, 3001, 1024], 128, "bf16", 0, seed=8101)
    # Second call on the same scratch, smaller: fewer heads and splits, d = 64.
    _case(2, 8, 2, [300, 1], 64, "f16", 3, seed=8102)


def test_noalloc_decode_refuses_more_than_its_scratch():
    import exact_io_aware_47_amd as fa
    q, kc, vc, table, sl = si.make_decode_inputs(8, 32, 8, [64] * 8, 128, "bf16", seed=8103)
    with pytest.raises(fa.FlashAttnError, match="FA_ERR_SCRATCH"):
        fa.decode_paged_noalloc(dev(q), dev(kc), dev(vc), dev(table), dev(sl), num_splits=1000)
