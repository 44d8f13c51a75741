"""fp64 CPU oracle for MLA paged-KV decode (test infrastructure only).

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may use it.
"""
from .mla_decode_oracle import (  # noqa: F401
    decode, decode_bruteforce, lse_merge, split_plan, plan_pieces,
    gather_request_kv, visible_count, attend_rows, fixed_cost_pages, rows_per_tile,
    num_pages, kv_append, mapped_keys, counted_view,
)
from .mla_fp8_oracle import (  # noqa: F401
    FP8_PAGE_BYTES, FP8_CODES_OFF, FP8_ROPE_OFF, FP8_SCALE_OFF, E4M3_TABLE,
    e4m3_decode, e4m3_encode, quantize_scale, quantize_row, dequant_page,
    gather_request_kv_fp8, decode_fp8, kv_append_fp8,
)
from .mla_sparse_oracle import (  # noqa: F401
    counted_entries, decode_sparse, decode_sparse_bruteforce, decode_sparse_fp8,
)
