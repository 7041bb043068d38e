"""CPU oracle for the scaled dot-product attention forward, in float64.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import or call this module.  The
library (``transformer_scaled_dot_flash_amd``) never does, and this module
imports nothing from the library.

What it computes is the plain definition, written out the slow, explicit
three-stage way, with no tiling and no online softmax:

    stage 1   S = scale * Q K^T                     (explicit score rows)
    stage 2   P = softmax_row(S + mask)             (three passes: max, sum, divide)
    stage 3   O = P V

Sources for each step (cited by page and section):

* The definition S = QK^T/sqrt(D), P = softmax_row(S + mask), O = PV and the
  causal rule "token i may not see j > i": learn-cuda-from-scratch Ch. 11
  "Attention", section 11.1; AIInfraGuide "Self-Attention" page, sections
  3.2-3.6.
* The scale is a multiplier applied to the raw dot product, as in the naive
  score kernel of section 11.3 of the Ch. 11 page; the caller supplies it
  (1/sqrt(d_k) in every workload, section 3.3 of the AIInfraGuide page).
* Softmax with the maximum subtracted, in three passes (find max; sum the
  exponentials; divide): AIInfraGuide page, section 7.2.
* Masked positions are set to minus infinity before the softmax and so get
  weight exactly 0: AIInfraGuide page, section 10.2 (the 4x4 example).
* Head mapping for MHA / MQA / GQA: q head h reads kv head h // group_size
  with group_size = H_q / H_kv: Ch. 11 page, section 11.8.1 and the unified
  kernel of section 11.11; AIInfraGuide page, section 9.3.
* Sliding window (Ch. 11 page, section 11.8.4: each token attends only to
  the most recent W tokens): with causal masking, row i sees keys j with
  i + off - W < j <= i + off, i.e. W keys ending at its own position.
* Packed variable-length batches (the flash_attn_varlen_func prefill form
  named in section 11.8.2 of the Ch. 11 page): every sequence is an
  independent attention problem; ``attention_varlen`` slices each one out of
  the packed token-major tensors and applies the same definition.

Readings where the pages leave a point open:

* Causal with T_q != T_kv (only T_q == T_kv appears on the pages): query row i
  is taken to sit at absolute position i + (T_kv - T_q), so it sees keys
  j <= i + T_kv - T_q ("bottom-right" alignment).  With T_q == T_kv this is
  exactly j <= i.  Callers never pass causal with T_q > T_kv, so every row
  sees at least one key.
* Inputs are whatever values the caller passes (float32 values or bfloat16
  values widened exactly); they are converted to float64 and nothing is
  rounded afterwards.  The output is float64.
* A query row that sees no key at all (only possible in a packed batch: an
  empty key range, or causal with the row before the first key) has output
  0; the softmax of an empty row is not defined on the pages.

Layout: Q [B, H_q, T_q, D], K and V [B, H_kv, T_kv, D], O [B, H_q, T_q, D].
"""
from __future__ import annotations

import numpy as np


def kv_head_for(h_q: int, H_q: int, H_kv: int) -> int:
    """KV head read by query head ``h_q``: h_q // (H_q / H_kv)."""
    if H_q % H_kv != 0:
        raise ValueError("H_q must be a multiple of H_kv")
    group_size = H_q // H_kv
    return h_q // group_size


def visible(rows: np.ndarray, T_q: int, T_kv: int, causal: bool, window: int = 0) -> np.ndarray:
    """Keep-mask [len(rows), T_kv]: True where query row i may see key j."""
    rows = np.asarray(rows, dtype=np.int64)
    j = np.arange(T_kv, dtype=np.int64)
    if not causal:
        return np.ones((rows.size, T_kv), dtype=bool)
    pos = rows[:, None] + (T_kv - T_q)  # absolute position of each query row
    keep = j[None, :] <= pos
    if window > 0:
        keep &= j[None, :] > pos - window
    return keep


def scores(q_rows: np.ndarray, k: np.ndarray, scale: float) -> np.ndarray:
    """Stage 1: S[i, j] = scale * sum_d q[i, d] k[j, d], in float64."""
    q_rows = np.asarray(q_rows, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    return np.float64(scale) * (q_rows @ k.T)


def softmax_rows(s: np.ndarray, keep: np.ndarray) -> np.ndarray:
    """Stage 2: row softmax of S with masked entries at -inf, three passes."""
    z = np.where(keep, s, -np.inf)
    m = np.max(z, axis=1, keepdims=True)          # pass 1: row maximum
    e = np.exp(z - m)                              # pass 2: exponentials ...
    total = np.sum(e, axis=1, keepdims=True)       # ... and their sum
    return e / total                               # pass 3: normalise


def weighted_sum(p: np.ndarray, v: np.ndarray) -> np.ndarray:
    """Stage 3: O[i, :] = sum_j P[i, j] v[j, :], in float64."""
    return p @ np.asarray(v, dtype=np.float64)


def attention_head(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float,
                   causal: bool, rows=None, return_p: bool = False, window: int = 0):
    """One (batch, q head) slice: q [T_q, D], k and v [T_kv, D].

    ``rows`` selects the query rows to compute (default: all).  Rows are
    independent of one another under the definition (the softmax is taken per
    row), so computing a subset gives exactly those rows of the full result.
    """
    T_q, T_kv = q.shape[0], k.shape[0]
    rows = np.arange(T_q) if rows is None else np.asarray(rows, dtype=np.int64)
    keep = visible(rows, T_q, T_kv, causal, window)
    seen = keep.any(axis=1)
    p = np.zeros((rows.size, T_kv), dtype=np.float64)
    if seen.any():
        s = scores(q[rows[seen]], k, scale)
        p[seen] = softmax_rows(s, keep[seen])
    o = weighted_sum(p, v) if T_kv else np.zeros((rows.size, q.shape[1]), dtype=np.float64)
    return (o, p) if return_p else o


def attention(Q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float,
              causal: bool, rows=None, heads=None, batches=None, window: int = 0) -> np.ndarray:
    """Full forward over [B, H, T, D] tensors; returns float64 O.

    ``rows``/``heads``/``batches`` restrict the output to a sample (used for
    workloads too large to compute whole on the CPU); the result then has
    shape [len(batches), len(heads), len(rows), D].
    """
    B, H_q, T_q, D = Q.shape
    Bk, H_kv, T_kv, Dk = K.shape
    if (Bk, Dk) != (B, D) or V.shape != K.shape:
        raise ValueError("Q, K, V shapes do not agree")
    if causal and T_q > T_kv:
        raise ValueError("causal attention needs T_q <= T_kv")
    batches = range(B) if batches is None else list(batches)
    heads = range(H_q) if heads is None else list(heads)
    row_sel = np.arange(T_q) if rows is None else np.asarray(rows, dtype=np.int64)
    out = np.empty((len(batches), len(heads), row_sel.size, D), dtype=np.float64)
    for bi, b in enumerate(batches):
        for hi, h in enumerate(heads):
            g = kv_head_for(h, H_q, H_kv)
            out[bi, hi] = attention_head(Q[b, h], K[b, g], V[b, g], scale, causal, row_sel,
                                         window=window)
    return out


def attention_varlen(q: np.ndarray, k: np.ndarray, v: np.ndarray, cu_q, cu_k, scale: float,
                     causal: bool, window: int = 0, seqs=None) -> np.ndarray:
    """Packed batch: q [total_q, H_q, D], k and v [total_k, H_kv, D] (token
    major); sequence b owns query rows cu_q[b]:cu_q[b+1] and key rows
    cu_k[b]:cu_k[b+1].  Returns float64 O [total_q, H_q, D]; rows of sequences
    not in ``seqs`` (default: all) are left 0."""
    total_q, H_q, D = q.shape
    H_kv = k.shape[1]
    out = np.zeros((total_q, H_q, D), dtype=np.float64)
    seqs = range(len(cu_q) - 1) if seqs is None else list(seqs)
    for b in seqs:
        qs, qe, ks, ke = int(cu_q[b]), int(cu_q[b + 1]), int(cu_k[b]), int(cu_k[b + 1])
        for h in range(H_q):
            g = kv_head_for(h, H_q, H_kv)
            out[qs:qe, h] = attention_head(q[qs:qe, h], k[ks:ke, g], v[ks:ke, g], scale, causal,
                                           window=window)
    return out
