"""CPU oracle for the fused QKV projection, in float64.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import or call this module.  The
library never does, and this module imports nothing from the library.

What it computes, in the two plain steps the pages describe
(learn-cuda-from-scratch Ch. 11 "Attention", section 11.2: Q, K and V are
three linear maps of the same input; section 11.8.1: query heads and kv heads
are column blocks of those maps, reshaped to one slice per head):

    1. Y = X W^T                       X [B*T, d_model], W [(H_q + 2 H_kv) D, d_model]
    2. split Y's columns into Q | K | V and reshape each to [B, H, T, D]
       (column h*D + d of a block is feature d of head h; row b*T + t is
       token t of sequence b)

Reading: the weight is stored one row per output feature (the layout of a
linear layer's weight), W_Q rows first, then W_K, then W_V.
"""
from __future__ import annotations

import numpy as np


def project(x: np.ndarray, w: np.ndarray) -> np.ndarray:
    """Step 1: Y = X W^T in float64, [B*T, N]."""
    return np.asarray(x, dtype=np.float64) @ np.asarray(w, dtype=np.float64).T


def split_heads(y: np.ndarray, B: int, T: int, H_q: int, H_kv: int, D: int):
    """Step 2: Y [B*T, (H_q + 2 H_kv) D] -> Q [B, H_q, T, D], K, V [B, H_kv, T, D]."""
    qn, kn = H_q * D, H_kv * D
    if y.shape != (B * T, qn + 2 * kn):
        raise ValueError("projection output has the wrong shape")

    def heads(block, H):
        return block.reshape(B, T, H, D).transpose(0, 2, 1, 3)

    return heads(y[:, :qn], H_q), heads(y[:, qn:qn + kn], H_kv), heads(y[:, qn + kn:], H_kv)


def qkv_project(x, w, B: int, T: int, H_q: int, H_kv: int, D: int):
    """Both steps: returns float64 (Q, K, V)."""
    return split_heads(project(x, w), B, T, H_q, H_kv, D)
