"""CPU oracle for paged KV-cache decode (test infrastructure only).

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may import
this package; the product package never does.
"""
from .pa_oracle import (  # noqa: F401
    cache_write,
    decode,
    decode_one,
    decode_one_online,
    decode_one_partitioned,
    gather_head,
    locate_kv,
    slot_to_block_offset,
    softmax,
)
