"""Grouped-query attention over a KV cache on AMD Instinct MI355X (gfx950).

The computation lives in libgqa.so (hand-written HIP kernels behind the C
ABI declared in include/gqa.h); this package is its thin ctypes binding
(``_binding``), the in-tree build script (``build``) and the seeded
synthetic-input generator (``inputs``).
"""
from ._binding import (  # noqa: F401
    GQA_BF16,
    GQA_F32,
    GQAError,
    HipEvent,
    gqa_abi_version,
    gqa_build_id,
    gqa_cross_attention,
    gqa_decode,
    gqa_decode_append,
    gqa_decode_append_noalloc,
    gqa_decode_append_int8,
    gqa_decode_append_paged,
    gqa_decode_int8,
    gqa_decode_paged,
    gqa_decode_paged_workspace_bytes,
    gqa_decode_workspace_bytes,
    gqa_kv_append,
    gqa_kv_append_paged,
    gqa_kv_append_int8,
    gqa_kv_append_rows,
    gqa_kv_quantize_int8,
    gqa_kv_cache_bytes,
    gqa_kv_project,
    gqa_kv_project_append,
    gqa_kv_project_workspace_bytes,
    gqa_last_error,
    gqa_meanpool_convert,
    gqa_prefill_causal,
    gqa_prefill_chunk,
    gqa_set_timing_events,
    header_symbols,
    load_library,
)
