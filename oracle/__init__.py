"""CPU float64 oracle for paged K/V-cache attention.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute anything in this package: only the test-suite, the smoke check of
``__graft_entry__`` and the CPU-baseline leg of ``bench.py`` use it.  It shares
no code, headers, tables or helpers with the HIP library; the two meet only in
the seeded input generators of the ``workloads`` package.
"""

from .pkv_oracle import (  # noqa: F401
    E4M3FN_MAX,
    attention_rows,
    attn_decode,
    attn_decode_shared_prefix,
    attn_decode_step,
    attn_prefill_block_causal,
    causal_layout,
    causal_layout_bounds,
    copy_slots,
    decode_bf16,
    decode_e4m3fn,
    e4m3fn_table,
    gather_logical,
    merge_states,
    prefill_visible_keys,
    rotate_rows,
    scatter_slots,
    visible_keys,
    window_evicted_tokens,
)
