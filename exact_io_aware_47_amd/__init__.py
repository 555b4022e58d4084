"""MI355X (gfx950) exact fused attention.

Hand-written HIP kernels behind a C ABI (``include/flash_attn.h``,
``libflash_attn_mi355x.so``); this package is its thin Python binding.
"""

from ._lib import (FA_BF16, FA_F16, FA_F32, FlashAttnError, bwd, bwd_phase, bwd_varlen, bwd_varlen_workspace_bytes,
                   bwd_workspace_bytes, decode_num_splits, decode_paged, decode_paged_noalloc, decode_workspace_bytes, fwd, fwd_fp8, fwd_fp8_workspace_bytes, fwd_varlen,
                   lib, prefill_paged, strerror)

__all__ = ["fwd", "fwd_fp8", "fwd_fp8_workspace_bytes", "bwd", "bwd_phase", "fwd_varlen", "bwd_varlen", "decode_paged", "decode_paged_noalloc", "prefill_paged", "bwd_workspace_bytes",
           "bwd_varlen_workspace_bytes", "decode_workspace_bytes", "decode_num_splits", "lib", "strerror",
           "FlashAttnError", "FA_F32", "FA_F16", "FA_BF16"]
