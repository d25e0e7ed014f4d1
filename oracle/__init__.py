"""Float64 CPU oracle for grouped-query attention: TEST INFRASTRUCTURE ONLY.

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The library (``grouped_query_decode_amd``)
never imports, links or calls it, and this package imports nothing from the
library: the two share no code.  See ``oracle/gqa_oracle.py`` for what each
function computes and which passage of the source pages it follows.
"""

from .gqa_oracle import (  # noqa: F401
    kv_group_of_head,
    group_map,
    attended_length,
    softmax_weights,
    attend_one_query,
    decode_ref,
    append_position,
    decode_append_ref,
    future_keys,
    prefill_causal_ref,
    chunk_attended_length,
    prefill_chunk_ref,
    gqkva_head_pair,
    gqkva_decode_ref,
    gqkva_prefill_causal_ref,
    meanpool_ref,
    kv_cache_values_per_token,
    kv_cache_bytes,
    kv_cache_reduction_factor,
    decode_flops,
    prefill_causal_flops,
)
