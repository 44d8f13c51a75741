"""MI355X (gfx950) paged-KV MLA decode attention.

The computation runs entirely in the HIP library libmla_decode.so (C ABI in
include/mla_decode.h); this package only marshals torch tensors into it.
"""
from .binding import (  # noqa: F401
    FP8_PAGE_BYTES, MLAError, combine, device_num_cus, fwd, fwd_fp8, fwd_inline_plan, fwd_noalloc, kv_append, kv_append_fp8,
    lib, metadata, num_parts, sparse_fwd, sparse_fwd_fp8, sparse_metadata, sparse_workspace_bytes, splitkv,
    splitkv_fp8, status_string, workspace_bytes,
)
