"""CPU oracle for decode over a paged KV cache, in float64.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import or call this module.  The
library never does, and this module imports nothing from the library.

What it computes: decode (one query token per sequence, every cached key
visible) where the keys and values of each sequence are not stored
contiguously but in fixed-size pages of a shared pool.  A block table maps
(sequence, token // page_size) to a physical page: learn-cuda-from-scratch
Ch. 11 "Attention", section 11.11 (KV-cache pages of 16 tokens, the block
table and the kernel's indirect K/V loads) and section 11.8.2 (decode as one
query vector against the whole cache).

The oracle is the plain definition written in two explicit steps:

    1. gather   K_b[j] = k_pages[block_table[b][j // page_size], g, j % page_size]
                for j = 0 .. seq_len_b - 1 (same for V), g = the q head's kv head
    2. attend   O[b, h] = softmax(scale * q[b, h] K_b^T) V_b    (the float64
                attention oracle of ``attention_fp64``, one query row)

Readings where the pages leave a point open (the library documents the same):

* Layout of a pool: [num_pages][H_kv][page_size][D], separate pools for K
  and V that share the block ids (the pages give the page contents -- K and
  V of page_size tokens for every kv head -- but no order within it).
* A sequence length is clamped to [0, max_pages * page_size]; a sequence of
  length 0 has no key and its output is defined as 0.
* A block id outside [0, num_pages) stands for a page of zeros.
"""
from __future__ import annotations

import numpy as np

from .attention_fp64 import attention_head, kv_head_for


def gather_sequence(pages: np.ndarray, block_row: np.ndarray, seq_len: int, page_size: int,
                    kv_head: int) -> np.ndarray:
    """Rows 0 .. seq_len-1 of one sequence and one kv head, [seq_len, D] float64."""
    num_pages, _, ps, D = pages.shape
    if ps != page_size:
        raise ValueError("page_size does not match the pool")
    j = np.arange(seq_len, dtype=np.int64)
    page = np.asarray(block_row, dtype=np.int64)[j // page_size]
    row = j % page_size
    ok = (page >= 0) & (page < num_pages)
    out = np.zeros((seq_len, D), dtype=np.float64)
    out[ok] = np.asarray(pages[page[ok], kv_head, row[ok]], dtype=np.float64)
    return out


def decode_paged(q: np.ndarray, k_pages: np.ndarray, v_pages: np.ndarray,
                 block_table: np.ndarray, seq_lens: np.ndarray, scale: float,
                 batches=None) -> np.ndarray:
    """q [B, H_q, D]; pools [num_pages, H_kv, page_size, D]; block_table
    [B, max_pages]; seq_lens [B].  Returns float64 O [len(batches), H_q, D]."""
    B, H_q, D = q.shape
    num_pages, H_kv, page_size, Dk = k_pages.shape
    if Dk != D or v_pages.shape != k_pages.shape:
        raise ValueError("pool shapes do not agree with q")
    max_pages = block_table.shape[1]
    t_max = max_pages * page_size
    batches = range(B) if batches is None else list(batches)
    out = np.zeros((len(batches), H_q, D), dtype=np.float64)
    for bi, b in enumerate(batches):
        L = int(min(max(int(seq_lens[b]), 0), t_max))
        if L == 0:
            continue  # no key: O = 0
        for h in range(H_q):
            g = kv_head_for(h, H_q, H_kv)
            k = gather_sequence(k_pages, block_table[b], L, page_size, g)
            v = gather_sequence(v_pages, block_table[b], L, page_size, g)
            out[bi, h] = attention_head(q[b, h][None, :], k, v, scale, False)[0]
    return out
