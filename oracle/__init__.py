"""CPU oracle for grouped-query attention over a KV cache.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path (the HIP library and
its Python binding) imports, calls or links anything in this package; only
the test-suite, the smoke check and the CPU-baseline leg of the benchmark do.

It is a plain, slow, obviously-correct float64 NumPy restatement of what the
hot path computes, written from the pages' description of the method:

* ``gqa_oracle``  -- the definitions (decode, causal prefill, cache append,
  paged-cache gather / decode / append, int8 cache quantisation / decode /
  append, chunked prefill over a cache, cross-attention, multi-row append,
  fused K/V projection + append, mean-pool conversion, KV-cache byte count,
  and the partition/merge model of the two-pass decode), vectorised with
  NumPy.
* ``bruteforce``  -- the same definitions as pure-Python scalar loops, for
  tiny inputs only; it derives the query-head -> KV-head grouping from the
  page's 1-based group formula independently of ``gqa_oracle``.

The two modules share no code with each other beyond the standard library
and NumPy, and none with the GPU path.
"""
from .gqa_oracle import (  # noqa: F401
    decode_ref,
    decode_weights_ref,
    prefill_causal_ref,
    kv_append_ref,
    meanpool_convert_ref,
    kv_cache_bytes,
    kv_head_of,
    paged_gather_ref,
    decode_paged_ref,
    kv_append_paged_ref,
    quantize_int8_ref,
    dequantize_int8_ref,
    decode_int8_ref,
    kv_append_int8_ref,
    prefill_chunk_ref,
    cross_attention_ref,
    kv_append_rows_ref,
    kv_project_ref,
    kv_project_append_ref,
    decode_partials_ref,
    combine_partials_ref,
)
