"""MI355X-native Medusa tree verification: C-ABI library (libmedusa.so) and its binding.

The four calls of one verification round, with the names of the C entry points:

    medusa_tree_compile   host tree compiler
    medusa_tree_attn      HIP tree attention (RoPE at P + depth, staged K/V rows)
    medusa_tree_attn_noalloc  the same with the library's own partials array
    medusa_accept         HIP greedy acceptance
    medusa_accept_typical HIP fast typical acceptance
    medusa_kv_compact     HIP winning-path K/V compaction
    medusa_head_candidates HIP Medusa head step and ranked candidate pool
"""
from ._binding import (  # noqa: F401
    BF16, F32, LIBRARY, MedusaError, STATUS, load, medusa_accept, medusa_accept_commit,
    medusa_accept_typical,
    medusa_accept_workspace_size, medusa_head_candidates, medusa_head_workspace_size,
    medusa_kv_compact, medusa_read_probe, medusa_read_probe_sink_size, medusa_tree_attn,
    medusa_tree_attn_noalloc, medusa_tree_attn_workspace_size, medusa_tree_budget, medusa_tree_compile,
)
