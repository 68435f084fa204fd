"""CPU oracle for the Star Attention hot path (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s
``cpu_baseline`` leg may import this package.  See ``star_oracle.py``.
"""
from .star_oracle import (  # noqa: F401
    NEG_INF, anchor_prefix_table, attend, blocks, chunks_of_block, dense_causal,
    document_frequency, kv_cache_entries, lse_merge, maxidf_score, maxidf_summaries,
    partial, partitions, phase1, phase1_block_keys, phase1_prefix, phase1_prefix_keys,
    phase1_prefix_rows, phase1_rows, phase2, pulsar_host_length, pulsar_prefix,
    remapped_anchor, rope, rope_theta, round_bf16, star_attention,
    rmsnorm, layer_projections, layer_output, attention_layer_phase1, causal_layer,
    star_context_per_host, star_context_layers,
)
