"""Streaming (online-softmax) attention forward and backward, and wide-row
split softmax, for AMD MI355X (gfx950).

The computation lives in the HIP library libattn.so (C ABI in
include/attn.h); this package is its Python binding plus the seeded
workload definitions used by the tests and the benchmark.
"""

from .attn import (  # noqa: F401
    ATTN_BF16,
    ATTN_E_HIP,
    ATTN_E_INVALID,
    ATTN_E_UNSUPPORTED,
    ATTN_F16,
    ATTN_F32,
    ATTN_OK,
    AttnError,
    attn_bwd,
    attn_decode_paged,
    attn_decode_paged_noalloc,
    attn_fwd,
    attn_fwd_dropout,
    attn_fwd_gqa,
    attn_fwd_masked,
    attn_fwd_raw,
    attn_fwd_stats,
    attn_fwd_varlen,
    attn_strerror,
    default_scale,
    online_merge,
    online_merge_batch,
    pack_mask,
    softmax_rows,
    softmax_rows_scratch_bytes,
)
