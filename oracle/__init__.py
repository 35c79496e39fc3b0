"""CPU oracle (float64) for paged decode attention.

TEST INFRASTRUCTURE ONLY: imported by the tests, ``__graft_entry__.smoke()``
and the CPU-baseline leg of ``bench.py``; never by the library.  It shares no
code with the GPU path.
"""
from .oracle import (attend, attended_range, copy_blocks, decode, decode_case, decode_sequence,
                     multi_query, multi_query_case, query_positions, reshape_and_cache, to_f64)

__all__ = ["attend", "attended_range", "copy_blocks", "decode", "decode_case", "decode_sequence",
           "multi_query", "multi_query_case", "query_positions", "reshape_and_cache", "to_f64"]
