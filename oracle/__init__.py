"""CPU oracle for Stream-Factorized Attention.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke`` and
the CPU-baseline leg of ``bench.py``; never by the library.
"""
from .sfa import (  # noqa: F401
    MIX,
    WITHIN,
    attention_backward_head,
    attention_rows,
    bf16_bits_to_f64,
    count_pairs,
    cyclic_replicate_ref,
    decode_append_ref,
    decode_ref,
    expand_ref,
    expanded_position,
    final_stream_rows_ref,
    gather_pages_ref,
    prefill_backward_ref,
    prefill_ref,
    scatter_pages_ref,
    useful_flops,
    visible,
)
