"""CPU float64 oracle for the attention forward.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py``, never by the library.
"""
from .attention_fp64 import (attention, attention_head, kv_head_for, scores, softmax_rows,
                        visible, weighted_sum)

__all__ = ["attention", "attention_head", "kv_head_for", "scores", "softmax_rows",
           "visible", "weighted_sum"]
