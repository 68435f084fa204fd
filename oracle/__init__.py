"""CPU oracle for the Star Attention hot path (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s
``cpu_baseline`` leg may import this package.  See ``star_oracle.py``.
"""
from .star_oracle import (  # noqa: F401
    NEG_INF, attend, blocks, dense_causal, kv_cache_entries, lse_merge,
    partial, partitions, phase1, phase1_block_keys, phase1_rows, phase2,
    rope, rope_theta, round_bf16, star_attention,
)
