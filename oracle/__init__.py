"""CPU float64 oracle for the attention forward.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py``, never by the library.
"""
from .attention_fp64 import (attention, attention_head, attention_varlen, kv_head_for, scores,
                             softmax_rows, visible, weighted_sum)
from .paged_fp64 import decode_paged, gather_sequence

__all__ = ["attention", "attention_head", "attention_varlen", "kv_head_for", "scores",
           "softmax_rows", "visible", "weighted_sum", "decode_paged", "gather_sequence"]
