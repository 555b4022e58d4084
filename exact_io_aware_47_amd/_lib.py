"""ctypes binding of ``libflash_attn_mi355x.so`` (argument marshalling only).

Every function here takes torch tensors, checks that they are dense device
tensors of one supported dtype, allocates missing outputs with torch (device
memory is torch's job), and passes raw pointers, sizes and torch's current HIP
stream to the C ABI declared in ``include/flash_attn.h``.  All arithmetic runs
in the library's HIP kernels; there is no other code path.  If the library is
not built, every call raises.
"""

from __future__ import annotations

import ctypes
import math
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libflash_attn_mi355x.so")

FA_F32, FA_F16, FA_BF16 = 0, 1, 2
_DTYPE_CODE = {torch.float32: FA_F32, torch.float16: FA_F16, torch.bfloat16: FA_BF16}

STATUS = {
    0: "FA_OK", 1: "FA_ERR_NULL", 2: "FA_ERR_SHAPE", 3: "FA_ERR_HEADDIM", 4: "FA_ERR_DTYPE",
    5: "FA_ERR_GQA", 6: "FA_ERR_BLOCKSIZE", 7: "FA_ERR_WORKSPACE", 8: "FA_ERR_LAUNCH", 9: "FA_ERR_SCALE", 10: "FA_ERR_ALIGN",
    11: "FA_ERR_SCRATCH",
}

_vp, _i, _f, _sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t

SIGNATURES = {
    "flash_attn_strerror": (ctypes.c_char_p, [_i]),
    "flash_attn_fwd": (_i, [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _f, _i, _i, _vp]),
    "flash_attn_bwd_workspace_bytes": (_sz, [_i, _i, _i, _i, _i, _i, _i]),
    "flash_attn_bwd": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                            _i, _i, _i, _i, _i, _i, _f, _i, _i, _vp, _sz, _vp]),
    "flash_attn_bwd_preprocess": (_i, [_vp, _vp, _vp, _i, _i, _i, _i, _i, _vp, _sz, _vp]),
    "flash_attn_bwd_dkdv": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _f, _i, _i, _vp, _sz, _vp]),
    "flash_attn_bwd_dq": (_i, [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _f, _i, _i, _vp, _sz, _vp]),
    "flash_attn_bwd_dq_rowterms": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _f, _i, _i,
                                        _vp, _sz, _vp]),
    "flash_attn_fwd_varlen": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _i, _f, _i, _i, _vp]),
    "flash_attn_bwd_varlen_workspace_bytes": (_sz, [_i, _i, _i, _i, _i, _i, _i, _i, _i]),
    "flash_attn_bwd_varlen": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                   _i, _i, _i, _i, _i, _i, _i, _i, _f, _i, _i, _vp, _sz, _vp]),
    "flash_attn_prefill_paged": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                      _i, _i, _i, _i, _i, _i, _i, _i, _f, _i, _i, _vp]),
    "flash_attn_fwd_fp8_workspace_bytes": (_sz, [_i, _i, _i, _i]),
    "flash_attn_fwd_fp8": (_i, [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _f, _f, _f, _f, _i, _vp, _sz, _vp]),
    "flash_attn_decode_num_splits": (_i, [_i, _i, _i, _i]),
    "flash_attn_decode_workspace_bytes": (_sz, [_i, _i, _i, _i, _i, _i, _i]),
    "flash_attn_decode_paged": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                     _i, _i, _i, _i, _i, _i, _i, _f, _i, _i, _vp, _sz, _vp]),
    "flash_attn_decode_paged_noalloc": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                             _i, _i, _i, _i, _i, _i, _i, _f, _i, _i, _vp]),
}

_lib = None


class FlashAttnError(RuntimeError):
    def __init__(self, code: int, what: str):
        self.code = code
        super().__init__(f"{what}: {STATUS.get(code, code)} ({strerror(code)})")


def lib() -> ctypes.CDLL:
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m exact_io_aware_47_amd.build`")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype, fn.argtypes = res, args
        _lib = handle
    return _lib


def strerror(code: int) -> str:
    return lib().flash_attn_strerror(code).decode()


def _check(code: int, what: str) -> None:
    if code != 0:
        raise FlashAttnError(code, what)


def _ptr(t: torch.Tensor | None):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _dense(name: str, t: torch.Tensor, dtype=None, ndim=None) -> torch.Tensor:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dimensions, got shape {tuple(t.shape)}")
    return t


def _out(name: str, t, shape, dtype, device: torch.device) -> torch.Tensor:
    """A caller-provided output checked against the shape the kernels write, or a new one."""
    if t is None:
        return torch.empty(shape, dtype=dtype, device=device)
    _dense(name, t, dtype)
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    return t


def _workspace(t, nbytes: int, device: torch.device) -> torch.Tensor:
    """A caller-provided workspace (its size is checked by the library), or a new one."""
    if t is None:
        return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)
    return _dense("workspace", t)


def _one_device(**tensors) -> torch.device:
    """The device of the first tensor; every other one must be on it."""
    devs = {n: t.device for n, t in tensors.items() if t is not None}
    first = next(iter(devs.values()))
    for n, dv in devs.items():
        if dv != first:
            raise ValueError(f"{n} is on {dv}, the other tensors on {first}")
    return first


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype not in _DTYPE_CODE:
        raise ValueError(f"unsupported dtype {t.dtype}; use float32, float16 or bfloat16")
    return _DTYPE_CODE[t.dtype]


def _default_scale(d: int, scale):
    return 1.0 / math.sqrt(d) if scale is None else float(scale)


def fwd(q, k, v, causal: bool = False, scale=None, out=None, lse=None):
    """O, LSE = attention(q, k, v).  q [B,Hq,Nq,d]; k, v [B,Hkv,Nk,d]."""
    _dense("q", q, ndim=4)
    _dense("k", k, q.dtype, 4)
    _dense("v", v, q.dtype, 4)
    B, Hq, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    if tuple(k.shape) != (B, Hkv, Nk, d) or tuple(v.shape) != (B, Hkv, Nk, d):
        raise ValueError(f"k/v shapes {tuple(k.shape)}, {tuple(v.shape)} do not match q {tuple(q.shape)}")
    dev = _one_device(q=q, k=k, v=v, out=out, lse=lse)
    out = _out("out", out, (B, Hq, Nq, d), q.dtype, dev)
    lse = _out("lse", lse, (B, Hq, Nq), torch.float32, dev)
    code = lib().flash_attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, Hq, Hkv, Nq, Nk, d,
                                _default_scale(d, scale), int(bool(causal)), _dtype_code(q), _stream(q.device))
    _check(code, "flash_attn_fwd")
    return out, lse


def bwd_workspace_bytes(B, Hq, Hkv, Nq, Nk, d, dtype_code) -> int:
    return int(lib().flash_attn_bwd_workspace_bytes(B, Hq, Hkv, Nq, Nk, d, dtype_code))


def bwd(q, k, v, out, dout, lse, causal: bool = False, scale=None, dq=None, dk=None, dv=None, workspace=None):
    """dQ, dK, dV of sum(O * dO) given the forward's O and LSE."""
    _dense("q", q, ndim=4)
    for name, t in (("k", k), ("v", v), ("out", out), ("dout", dout)):
        _dense(name, t, q.dtype, 4)
    _dense("lse", lse, torch.float32, 3)
    B, Hq, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    if tuple(k.shape) != (B, Hkv, Nk, d) or tuple(v.shape) != (B, Hkv, Nk, d):
        raise ValueError(f"k/v shapes {tuple(k.shape)}, {tuple(v.shape)} do not match q {tuple(q.shape)}")
    if out.shape != q.shape or dout.shape != q.shape or tuple(lse.shape) != (B, Hq, Nq):
        raise ValueError(f"out {tuple(out.shape)}, dout {tuple(dout.shape)} or lse {tuple(lse.shape)} "
                         f"do not match q {tuple(q.shape)}")
    dev = _one_device(q=q, k=k, v=v, out=out, dout=dout, lse=lse, dq=dq, dk=dk, dv=dv, workspace=workspace)
    dq = _out("dq", dq, q.shape, q.dtype, dev)
    dk = _out("dk", dk, k.shape, q.dtype, dev)
    dv = _out("dv", dv, v.shape, q.dtype, dev)
    code_dt = _dtype_code(q)
    workspace = _workspace(workspace, bwd_workspace_bytes(B, Hq, Hkv, Nq, Nk, d, code_dt), dev)
    code = lib().flash_attn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(dout), _ptr(lse), _ptr(dq), _ptr(dk),
                                _ptr(dv), B, Hq, Hkv, Nq, Nk, d, _default_scale(d, scale), int(bool(causal)), code_dt,
                                _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(q.device))
    _check(code, "flash_attn_bwd")
    return dq, dk, dv


def bwd_phase(phase: str, q, k, v, out, dout, lse, dq, dk, dv, workspace, causal: bool = False, scale=None):
    """Run one backward phase ('preprocess', 'dkdv', 'dq', or 'dq_rowterms':
    dQ computing the row terms into the workspace itself, in place of
    'preprocess') on torch's current stream; the outputs and the workspace are
    caller-allocated.  Arguments not used by the phase may be None."""
    given = dict(q=q, k=k, v=v, out=out, dout=dout, lse=lse, dq=dq, dk=dk, dv=dv, workspace=workspace)
    for name, t in given.items():
        if t is not None:
            _dense(name, t)
    _one_device(**given)
    ref = q if q is not None else out
    B, Hq, Nq, d = ref.shape
    Hkv, Nk = (k.shape[1], k.shape[2]) if k is not None else (Hq, Nq)
    code_dt = _dtype_code(ref)
    ws = (_ptr(workspace), workspace.numel() * workspace.element_size())
    sc = _default_scale(d, scale)
    L = lib()
    if phase == "preprocess":
        code = L.flash_attn_bwd_preprocess(_ptr(out), _ptr(dout), _ptr(lse), B, Hq, Nq, d, code_dt, *ws,
                                           _stream(ref.device))
    elif phase == "dkdv":
        code = L.flash_attn_bwd_dkdv(_ptr(q), _ptr(k), _ptr(v), _ptr(dout), _ptr(dk), _ptr(dv), B, Hq, Hkv, Nq, Nk,
                                     d, sc, int(bool(causal)), code_dt, *ws, _stream(ref.device))
    elif phase == "dq":
        code = L.flash_attn_bwd_dq(_ptr(q), _ptr(k), _ptr(v), _ptr(dout), _ptr(dq), B, Hq, Hkv, Nq, Nk, d, sc,
                                   int(bool(causal)), code_dt, *ws, _stream(ref.device))
    elif phase == "dq_rowterms":
        code = L.flash_attn_bwd_dq_rowterms(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(dout), _ptr(lse), _ptr(dq),
                                            B, Hq, Hkv, Nq, Nk, d, sc, int(bool(causal)), code_dt, *ws,
                                            _stream(ref.device))
    else:
        raise ValueError(f"unknown backward phase {phase!r}")
    _check(code, f"flash_attn_bwd_{phase}")


def _packed(q, k, cu_q, cu_k, hq, hkv, max_seqlen_q, max_seqlen_k):
    """Sizes of a packed batch: q [hq*total_q, d], k [hkv*total_k, d], cu_* [B+1] int32."""
    _dense("q", q, ndim=2)
    _dense("k", k, q.dtype, 2)
    _dense("cu_q", cu_q, torch.int32, 1)
    _dense("cu_k", cu_k, torch.int32, 1)
    if cu_q.numel() != cu_k.numel() or cu_q.numel() < 2:
        raise ValueError(f"cu_q and cu_k must both have B + 1 >= 2 entries, got {cu_q.numel()} and {cu_k.numel()}")
    if q.shape[0] % hq or k.shape[0] % hkv or q.shape[1] != k.shape[1]:
        raise ValueError(f"packed shapes q {tuple(q.shape)} / k {tuple(k.shape)} do not match Hq={hq}, Hkv={hkv}")
    return cu_q.numel() - 1, q.shape[0] // hq, k.shape[0] // hkv, q.shape[1], int(max_seqlen_q), int(max_seqlen_k)


def fwd_varlen(q, k, v, cu_q, cu_k, hq: int, hkv: int, max_seqlen_q: int, max_seqlen_k: int, causal: bool = False,
               scale=None, out=None, lse=None):
    """O, LSE of a packed batch.  q [hq*total_q, d]; k, v [hkv*total_k, d];
    head h of sequence b occupies rows H*cu[b] + h*n_b ... (+ n_b)."""
    B, tq, tk, d, mq, mk = _packed(q, k, cu_q, cu_k, hq, hkv, max_seqlen_q, max_seqlen_k)
    _dense("v", v, q.dtype, 2)
    if v.shape != k.shape:
        raise ValueError(f"v shape {tuple(v.shape)} does not match k {tuple(k.shape)}")
    dev = _one_device(q=q, k=k, v=v, cu_q=cu_q, cu_k=cu_k, out=out, lse=lse)
    out = _out("out", out, q.shape, q.dtype, dev)
    lse = _out("lse", lse, (q.shape[0],), torch.float32, dev)
    code = lib().flash_attn_fwd_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(cu_q), _ptr(cu_k),
                                       B, hq, hkv, tq, tk, mq, mk, d, _default_scale(d, scale), int(bool(causal)),
                                       _dtype_code(q), _stream(q.device))
    _check(code, "flash_attn_fwd_varlen")
    return out, lse


def bwd_varlen_workspace_bytes(B, hq, hkv, total_q, total_k, max_seqlen_q, max_seqlen_k, d, dtype_code) -> int:
    return int(lib().flash_attn_bwd_varlen_workspace_bytes(B, hq, hkv, total_q, total_k, max_seqlen_q, max_seqlen_k,
                                                           d, dtype_code))


def bwd_varlen(q, k, v, out, dout, lse, cu_q, cu_k, hq: int, hkv: int, max_seqlen_q: int, max_seqlen_k: int,
               causal: bool = False, scale=None, dq=None, dk=None, dv=None, workspace=None):
    """dQ, dK, dV of a packed batch (layout as in fwd_varlen)."""
    B, tq, tk, d, mq, mk = _packed(q, k, cu_q, cu_k, hq, hkv, max_seqlen_q, max_seqlen_k)
    for name, t in (("v", v), ("out", out), ("dout", dout)):
        _dense(name, t, q.dtype, 2)
    _dense("lse", lse, torch.float32, 1)
    if v.shape != k.shape or out.shape != q.shape or dout.shape != q.shape or lse.shape[0] != q.shape[0]:
        raise ValueError(f"v {tuple(v.shape)}, out {tuple(out.shape)}, dout {tuple(dout.shape)} or lse "
                         f"{tuple(lse.shape)} do not match q {tuple(q.shape)} / k {tuple(k.shape)}")
    dev = _one_device(q=q, k=k, v=v, out=out, dout=dout, lse=lse, cu_q=cu_q, cu_k=cu_k, dq=dq, dk=dk, dv=dv,
                      workspace=workspace)
    dq = _out("dq", dq, q.shape, q.dtype, dev)
    dk = _out("dk", dk, k.shape, q.dtype, dev)
    dv = _out("dv", dv, v.shape, q.dtype, dev)
    code_dt = _dtype_code(q)
    workspace = _workspace(workspace, bwd_varlen_workspace_bytes(B, hq, hkv, tq, tk, mq, mk, d, code_dt), dev)
    code = lib().flash_attn_bwd_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(dout), _ptr(lse), _ptr(dq),
                                       _ptr(dk), _ptr(dv), _ptr(cu_q), _ptr(cu_k), B, hq, hkv, tq, tk, mq, mk, d,
                                       _default_scale(d, scale), int(bool(causal)), code_dt, _ptr(workspace),
                                       workspace.numel() * workspace.element_size(), _stream(q.device))
    _check(code, "flash_attn_bwd_varlen")
    return dq, dk, dv


def prefill_paged(q, k_cache, v_cache, block_table, seq_lens, causal: bool = True, scale=None, out=None, lse=None):
    """Attention of a chunk of queries (the last Nq positions of each sequence)
    over a paged cache.  q [B,Hq,Nq,d]; k_cache, v_cache
    [num_blocks,Hkv,block_size,d]; block_table [B,max_blocks] int32;
    seq_lens [B] int32 (cached tokens, the chunk's own included)."""
    _dense("q", q, ndim=4)
    _dense("k_cache", k_cache, q.dtype, 4)
    _dense("v_cache", v_cache, q.dtype, 4)
    _dense("block_table", block_table, torch.int32, 2)
    _dense("seq_lens", seq_lens, torch.int32, 1)
    B, Hq, Nq, d = q.shape
    num_blocks, Hkv, bs, _ = k_cache.shape
    if v_cache.shape != k_cache.shape or k_cache.shape[3] != d or block_table.shape[0] != B or \
            seq_lens.shape[0] != B:
        raise ValueError("cache, table or lengths do not match q")
    dev = _one_device(q=q, k_cache=k_cache, v_cache=v_cache, block_table=block_table, seq_lens=seq_lens, out=out,
                      lse=lse)
    out = _out("out", out, q.shape, q.dtype, dev)
    lse = _out("lse", lse, (B, Hq, Nq), torch.float32, dev)
    code = lib().flash_attn_prefill_paged(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table), _ptr(seq_lens),
                                          _ptr(out), _ptr(lse), B, Hq, Hkv, Nq, d, bs, block_table.shape[1], num_blocks,
                                          _default_scale(d, scale), int(bool(causal)), _dtype_code(q),
                                          _stream(q.device))
    _check(code, "flash_attn_prefill_paged")
    return out, lse


def fwd_fp8_workspace_bytes(B, Hkv, Nk, d) -> int:
    return int(lib().flash_attn_fwd_fp8_workspace_bytes(B, Hkv, Nk, d))


def fwd_fp8(q, k, v, q_descale=1.0, k_descale=1.0, v_descale=1.0, causal: bool = False, scale=None, out=None,
            lse=None, workspace=None):
    """O (bf16), LSE of FP8 inputs: q [B,Hq,Nq,d], k, v [B,Hkv,Nk,d] as
    torch.float8_e4m3fn (or uint8 codes), each times its descale."""
    _dense("q", q, ndim=4)
    for name, t in (("k", k), ("v", v)):
        _dense(name, t, q.dtype, 4)
    if q.dtype not in (torch.float8_e4m3fn, torch.uint8):
        raise ValueError(f"fp8 inputs must be torch.float8_e4m3fn or uint8 codes, got {q.dtype}")
    B, Hq, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    if tuple(k.shape) != (B, Hkv, Nk, d) or tuple(v.shape) != (B, Hkv, Nk, d):
        raise ValueError(f"k/v shapes {tuple(k.shape)}, {tuple(v.shape)} do not match q {tuple(q.shape)}")
    dev = _one_device(q=q, k=k, v=v, out=out, lse=lse, workspace=workspace)
    out = _out("out", out, (B, Hq, Nq, d), torch.bfloat16, dev)
    lse = _out("lse", lse, (B, Hq, Nq), torch.float32, dev)
    workspace = _workspace(workspace, fwd_fp8_workspace_bytes(B, Hkv, Nk, d), dev)
    code = lib().flash_attn_fwd_fp8(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, Hq, Hkv, Nq, Nk, d,
                                    _default_scale(d, scale), float(q_descale), float(k_descale), float(v_descale),
                                    int(bool(causal)), _ptr(workspace), workspace.numel() * workspace.element_size(),
                                    _stream(q.device))
    _check(code, "flash_attn_fwd_fp8")
    return out, lse


def decode_num_splits(B, Hkv, max_blocks_per_seq, block_size=16) -> int:
    return int(lib().flash_attn_decode_num_splits(B, Hkv, max_blocks_per_seq, block_size))


def decode_workspace_bytes(B, Hq, Hkv, d, max_blocks_per_seq, block_size=16, num_splits=0) -> int:
    return int(lib().flash_attn_decode_workspace_bytes(B, Hq, Hkv, d, max_blocks_per_seq, block_size, num_splits))


def decode_paged(q, k_cache, v_cache, block_table, seq_lens, scale=None, num_splits: int = 0, out=None, lse=None,
                 workspace=None, want_lse: bool = True):
    """One-token split-KV decode over a paged cache.  q [B,Hq,d];
    k_cache, v_cache [num_blocks,Hkv,block_size,d]; block_table [B,max_blocks]
    int32; seq_lens [B] int32."""
    _dense("q", q, ndim=3)
    _dense("k_cache", k_cache, q.dtype, 4)
    _dense("v_cache", v_cache, q.dtype, 4)
    _dense("block_table", block_table, torch.int32, 2)
    _dense("seq_lens", seq_lens, torch.int32, 1)
    B, Hq, d = q.shape
    num_blocks, Hkv, bs, _ = k_cache.shape
    max_blocks = block_table.shape[1]
    if v_cache.shape != k_cache.shape or k_cache.shape[3] != d or block_table.shape[0] != B or \
            seq_lens.shape[0] != B:
        raise ValueError("cache, table or lengths do not match q")
    dev = _one_device(q=q, k_cache=k_cache, v_cache=v_cache, block_table=block_table, seq_lens=seq_lens, out=out,
                      lse=lse, workspace=workspace)
    out = _out("out", out, q.shape, q.dtype, dev)
    if lse is not None or want_lse:
        lse = _out("lse", lse, (B, Hq), torch.float32, dev)
    workspace = _workspace(workspace, decode_workspace_bytes(B, Hq, Hkv, d, max_blocks, bs, num_splits), dev)
    code = lib().flash_attn_decode_paged(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table), _ptr(seq_lens),
                                         _ptr(out), _ptr(lse), B, Hq, Hkv, d, bs, max_blocks, num_blocks,
                                         _default_scale(d, scale), int(num_splits), _dtype_code(q),
                                         _ptr(workspace), workspace.numel() * workspace.element_size(),
                                         _stream(q.device))
    _check(code, "flash_attn_decode_paged")
    return out, lse


DECODE_SCRATCH_BYTES = 8 << 20  # FLASH_ATTN_DECODE_SCRATCH_BYTES


def decode_paged_noalloc(q, k_cache, v_cache, block_table, seq_lens, scale=None, num_splits: int = 0, out=None,
                         lse=None, want_lse: bool = True):
    """decode_paged without a workspace: the library's fixed per-GPU scratch
    area holds the split records (flash_attn_decode_paged_noalloc).  Pass
    ``out`` (and ``lse``) to allocate nothing at all; calls that overlap on
    one GPU race."""
    _dense("q", q, ndim=3)
    _dense("k_cache", k_cache, q.dtype, 4)
    _dense("v_cache", v_cache, q.dtype, 4)
    _dense("block_table", block_table, torch.int32, 2)
    _dense("seq_lens", seq_lens, torch.int32, 1)
    B, Hq, d = q.shape
    num_blocks, Hkv, bs, _ = k_cache.shape
    max_blocks = block_table.shape[1]
    if v_cache.shape != k_cache.shape or k_cache.shape[3] != d or block_table.shape[0] != B or \
            seq_lens.shape[0] != B:
        raise ValueError("cache, table or lengths do not match q")
    dev = _one_device(q=q, k_cache=k_cache, v_cache=v_cache, block_table=block_table, seq_lens=seq_lens, out=out,
                      lse=lse)
    out = _out("out", out, q.shape, q.dtype, dev)
    if lse is not None or want_lse:
        lse = _out("lse", lse, (B, Hq), torch.float32, dev)
    code = lib().flash_attn_decode_paged_noalloc(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table),
                                                 _ptr(seq_lens), _ptr(out), _ptr(lse), B, Hq, Hkv, d, bs, max_blocks,
                                                 num_blocks, _default_scale(d, scale), int(num_splits),
                                                 _dtype_code(q), _stream(q.device))
    _check(code, "flash_attn_decode_paged_noalloc")
    return out, lse
