"""CPU float64 oracle for paged decode attention.

TEST INFRASTRUCTURE: only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import it. The HIP library never does.
"""
from .attention_f64 import (  # noqa: F401
    attend_one,
    attended_range,
    decode_attention,
    decode_attention_sharded,
    gather_rows,
    kv_head_of,
    merge_states,
    relative_l2,
    relative_l2_per_row,
    round_to,
    shard_state,
)
from .paged_cache import append_kv  # noqa: F401,E402
from .multi_query import prefill_attention  # noqa: F401,E402
