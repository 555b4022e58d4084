"""The Python binding rejects caller-provided outputs and workspaces that do
not fit what the kernels write, before anything is launched.

The C ABI receives bare pointers and cannot see an output's size, so the
binding compares every provided tensor with the shape the call writes.
"""

from __future__ import annotations

import pytest
import torch

pytestmark = pytest.mark.gpu


def _fa():
    import exact_io_aware_47_amd as fa
    return fa


def _t(*shape, dtype=torch.bfloat16):
    return torch.zeros(shape, dtype=dtype, device="cuda")


def test_fwd_rejects_misshaped_outputs():
    fa = _fa()
    q, k, v = _t(1, 2, 64, 64), _t(1, 2, 64, 64), _t(1, 2, 64, 64)
    with pytest.raises(ValueError, match="out must have shape"):
        fa.fwd(q, k, v, out=_t(1, 2, 63, 64))
    with pytest.raises(ValueError, match="lse must have shape"):
        fa.fwd(q, k, v, lse=_t(1, 2, 32, dtype=torch.float32))
    with pytest.raises(ValueError, match="must be torch.float32"):
        fa.fwd(q, k, v, lse=_t(1, 2, 64))
    with pytest.raises(ValueError, match="cpu"):
        fa.fwd(q, k, v, out=torch.zeros(1, 2, 64, 64, dtype=torch.bfloat16))


def test_bwd_rejects_misshaped_inputs_and_outputs():
    fa = _fa()
    q, k, v = _t(1, 4, 64, 64), _t(1, 2, 96, 64), _t(1, 2, 96, 64)
    o, do, lse = _t(1, 4, 64, 64), _t(1, 4, 64, 64), _t(1, 4, 64, dtype=torch.float32)
    with pytest.raises(ValueError, match="do not match q"):
        fa.bwd(q, k, v, o, _t(1, 4, 32, 64), lse)
    with pytest.raises(ValueError, match="do not match q"):
        fa.bwd(q, k, _t(1, 2, 95, 64), o, do, lse)
    with pytest.raises(ValueError, match="dk must have shape"):
        fa.bwd(q, k, v, o, do, lse, dk=_t(1, 4, 96, 64))
    with pytest.raises(ValueError, match="dq must have shape"):
        fa.bwd(q, k, v, o, do, lse, dq=_t(1, 4, 64, 32))


def test_varlen_rejects_misshaped_outputs():
    fa = _fa()
    cu = torch.tensor([0, 10, 30], dtype=torch.int32, device="cuda")
    q, k, v = _t(2 * 30, 64), _t(30, 64), _t(30, 64)
    with pytest.raises(ValueError, match="lse must have shape"):
        fa.fwd_varlen(q, k, v, cu, cu, 2, 1, 20, 20, lse=_t(30, dtype=torch.float32))
    o, lse = _t(60, 64), _t(60, dtype=torch.float32)
    with pytest.raises(ValueError, match="dv must have shape"):
        fa.bwd_varlen(q, k, v, o, o, lse, cu, cu, 2, 1, 20, 20, dv=_t(60, 64))


def test_paged_calls_reject_misshaped_outputs():
    fa = _fa()
    kc, vc = _t(8, 2, 16, 64), _t(8, 2, 16, 64)
    table = torch.zeros(2, 4, dtype=torch.int32, device="cuda")
    lens = torch.tensor([5, 40], dtype=torch.int32, device="cuda")
    with pytest.raises(ValueError, match="lse must have shape"):
        fa.decode_paged(_t(2, 4, 64), kc, vc, table, lens, lse=_t(2, 2, dtype=torch.float32))
    with pytest.raises(ValueError, match="do not match q"):
        fa.decode_paged(_t(2, 4, 128), kc, vc, table, lens)
    with pytest.raises(ValueError, match="out must have shape"):
        fa.prefill_paged(_t(2, 4, 3, 64), kc, vc, table, lens, out=_t(2, 4, 4, 64))


def test_fp8_rejects_misshaped_outputs():
    fa = _fa()
    q = torch.zeros(1, 2, 64, 64, dtype=torch.uint8, device="cuda")
    with pytest.raises(ValueError, match="out must have shape"):
        fa.fwd_fp8(q, q, q, out=_t(1, 2, 64, 32))
    with pytest.raises(ValueError, match="must be torch.bfloat16"):
        fa.fwd_fp8(q, q, q, out=_t(1, 2, 64, 64, dtype=torch.float16))
