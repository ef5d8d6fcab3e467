"""MI355X (gfx950) paged GQA decode attention: Python binding of libpaged_attn.so.

The C ABI (include/paged_attn.h) exports kv_append, paged_decode_attn,
paged_verify_attn, paged_decode_attn_split, lse_merge, paged_attn_balanced and
paged_attn_balanced_merge (with paged_attn_balanced_workspace_bytes and
paged_attn_balanced_workgroups), paged_decode_step, paged_decode_step_noalloc, kv_copy_blocks, kv_append_quant,
paged_multi_query_attn, kv_gather, paged_split_workspace_bytes and paged_status_string; this package exposes the same
names over torch tensors.  Importing it fails if the library has not been built
(``python paged_gqa_decode_kv_amd/build.py``).
"""
from ._binding import (  # noqa: F401
    LIB_PATH, PA_BF16, PA_F32, PA_FP8, PA_I8, PagedAttnError, kv_append, kv_gather, lib, lse_merge,
    make_dims, pa_dims, paged_decode_attn, paged_decode_attn_split, paged_split_workspace_bytes,
    paged_status_string, paged_verify_attn, paged_attn_balanced, paged_attn_balanced_workgroups,
    paged_attn_balanced_workspace_bytes, paged_attn_balanced_merge, paged_decode_step,
    paged_decode_step_noalloc, PA_NOALLOC_SCRATCH_BYTES,
    kv_copy_blocks, kv_append_quant, paged_multi_query_attn)
