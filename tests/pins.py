"""Checks that pin the CPU oracle to facts fixed by the pages and by mathematics.

Each ``pin_*`` function raises AssertionError when the oracle disagrees with
the fact it encodes.  They call the oracle through its module
(``oracle.attention_fp64``) at call time, so a test can plant a mistake in one of
the oracle's functions and confirm that some pin catches it.

None of these restate the oracle's own formula: they use closed forms,
special cases that reduce to a library routine, brute force in plain Python
scalars on tiny inputs, invariants of the definition, the worked examples
printed on the pages, and a second formulation of the same result (the
online softmax and block merge) that the pages state separately.
"""
from __future__ import annotations

import math
from pathlib import Path

import numpy as np
from scipy import special

import oracle.attention_fp64 as A

GOLDEN = Path(__file__).resolve().parent / "golden"


def _rng(seed):
    return np.random.default_rng(seed)


def _close(a, b, tol, what):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} != {b.shape}"
    assert np.all(np.isfinite(a)), f"{what}: non-finite values"
    err = float(np.max(np.abs(a - b))) if a.size else 0.0
    assert err <= tol, f"{what}: max abs error {err:.3e} > {tol:.1e}"


# --- softmax rows are probability distributions ------------------------------
def pin_rows_sum_to_one():
    """Each softmax row sums to 1, weights are >= 0 and masked ones are exactly 0
    (AIInfraGuide page, sections 3.4 and 10.2)."""
    r = _rng(1)
    for causal, T_q, T_kv in [(False, 7, 7), (True, 9, 9), (True, 5, 12), (False, 4, 11)]:
        q = r.standard_normal((T_q, 16))
        k = r.standard_normal((T_kv, 16))
        v = r.standard_normal((T_kv, 16))
        _, p = A.attention_head(q, k, v, 0.25, causal, return_p=True)
        assert p.shape == (T_q, T_kv), "softmax rows have the wrong shape"
        _close(p.sum(axis=1), np.ones(T_q), 1e-12, "row sums")
        assert np.all(p >= 0), "negative weight"
        if causal:
            off = T_kv - T_q
            i, j = np.indices((T_q, T_kv))
            assert np.all(p[j > i + off] == 0), "masked key has nonzero weight"


# --- causal row 0 sees only key 0 ----------------------------------------------
def pin_causal_row0_is_v0():
    """With T_q == T_kv, causal row 0 sees key 0 alone, so O[0] == V[0] exactly
    (Ch. 11 page, section 11.1; AIInfraGuide page, section 10.2)."""
    r = _rng(2)
    Q = r.standard_normal((2, 4, 10, 8))
    K = r.standard_normal((2, 2, 10, 8))
    V = r.standard_normal((2, 2, 10, 8))
    O = A.attention(Q, K, V, 0.3, True)
    for b in range(2):
        for h in range(4):
            assert np.array_equal(O[b, h, 0], V[b, h // 2, 0]), "causal O[0] != V[0]"


# --- Q = 0 gives uniform weights over the visible keys -----------------------
def pin_zero_query_gives_mean():
    """Q = 0 makes every score 0, so the weights are uniform over the visible
    keys: causal row i is the mean of V[0..i+off], non-causal rows the mean of
    all of V (closed form of the softmax of a constant row)."""
    r = _rng(3)
    for causal, T_q, T_kv in [(True, 12, 12), (True, 5, 12), (False, 6, 9)]:
        Q = np.zeros((1, 2, T_q, 8))
        K = r.standard_normal((1, 1, T_kv, 8))
        V = r.standard_normal((1, 1, T_kv, 8))
        O = A.attention(Q, K, V, 0.5, causal)
        if causal:
            off = T_kv - T_q
            csum = np.cumsum(V[0, 0], axis=0)
            want = np.stack([csum[i + off] / (i + off + 1) for i in range(T_q)])
        else:
            want = np.broadcast_to(V[0, 0].mean(axis=0), (T_q, 8))
        for h in range(2):
            _close(O[0, h], want, 1e-12, f"Q=0 mean (causal={causal}, T_q={T_q}, T_kv={T_kv})")


# --- head mapping --------------------------------------------------------------
def pin_gqa_is_repeated_mha():
    """GQA equals MHA with each kv head repeated group_size times, consecutive
    q heads sharing one kv head (Ch. 11 page, sections 11.8.1 and 11.11;
    AIInfraGuide page, section 9.3: g = h gives MHA, g = 1 gives MQA)."""
    r = _rng(4)
    for H_q, H_kv in [(8, 2), (6, 3), (4, 1), (4, 4)]:
        Q = r.standard_normal((2, H_q, 6, 8))
        K = r.standard_normal((2, H_kv, 6, 8))
        V = r.standard_normal((2, H_kv, 6, 8))
        G = H_q // H_kv
        Kr = np.repeat(K, G, axis=1)
        Vr = np.repeat(V, G, axis=1)
        for causal in (False, True):
            got = A.attention(Q, K, V, 0.4, causal)
            mha = A.attention(Q, Kr, Vr, 0.4, causal)
            assert np.array_equal(got, mha), f"GQA {H_q}/{H_kv} != repeated MHA"
    # Which kv head: V constant per kv head makes O reveal the head index.
    Q = r.standard_normal((1, 6, 5, 4))
    K = r.standard_normal((1, 3, 5, 4))
    V = np.zeros((1, 3, 5, 4))
    for g in range(3):
        V[0, g] = g + 1.0
    O = A.attention(Q, K, V, 1.0, False)
    for h in range(6):
        _close(O[0, h], np.full((5, 4), h // 2 + 1.0), 1e-12, f"q head {h} kv head")


# --- tiny cases in closed form -------------------------------------------------
def pin_single_key():
    """One key: every row's weight is 1 and O == V[0] for any Q, K."""
    r = _rng(5)
    Q = r.standard_normal((1, 2, 7, 8))
    K = r.standard_normal((1, 2, 1, 8))
    V = r.standard_normal((1, 2, 1, 8))
    O = A.attention(Q, K, V, 0.7, False)
    for h in range(2):
        _close(O[0, h], np.broadcast_to(V[0, h, 0], (7, 8)), 0.0, "single key")


def pin_two_keys_sigmoid():
    """Two keys, non-causal: weight of key 0 is sigmoid(scale * q.(k0 - k1)),
    so O_i = s V0 + (1 - s) V1 (closed form of a 2-way softmax)."""
    r = _rng(6)
    Q = r.standard_normal((1, 1, 9, 8))
    K = r.standard_normal((1, 1, 2, 8))
    V = r.standard_normal((1, 1, 2, 8))
    scale = 0.35
    O = A.attention(Q, K, V, scale, False)
    q = Q[0, 0]
    k0, k1 = K[0, 0, 0], K[0, 0, 1]
    s = special.expit(scale * (q @ (k0 - k1)))
    want = s[:, None] * V[0, 0, 0][None, :] + (1 - s)[:, None] * V[0, 0, 1][None, :]
    _close(O[0, 0], want, 1e-13, "two-key sigmoid")


def _brute_force(Q, K, V, scale, causal):
    """Plain-Python scalar loops: the definition with no numpy at all."""
    B, H_q, T_q, D = len(Q), len(Q[0]), len(Q[0][0]), len(Q[0][0][0])
    H_kv, T_kv = len(K[0]), len(K[0][0])
    G = H_q // H_kv
    out = [[[[0.0] * D for _ in range(T_q)] for _ in range(H_q)] for _ in range(B)]
    for b in range(B):
        for h in range(H_q):
            g = h // G
            for i in range(T_q):
                w = []
                for j in range(T_kv):
                    if causal and j > i + (T_kv - T_q):
                        w.append(0.0)
                        continue
                    dot = 0.0
                    for d in range(D):
                        dot += Q[b][h][i][d] * K[b][g][j][d]
                    w.append(math.exp(scale * dot))
                tot = math.fsum(w)
                for d in range(D):
                    out[b][h][i][d] = math.fsum(w[j] * V[b][g][j][d] for j in range(T_kv)) / tot
    return out


def pin_brute_force_worked_shape():
    """The worked shape example of AIInfraGuide section 5 (batch 1, 8 heads,
    6 tokens, head_dim 64, scores divided by sqrt(64) = 8), plus a GQA and a
    chunked-causal case, against scalar brute force."""
    r = _rng(7)
    cases = [
        ((1, 8, 6, 64), (1, 8, 6, 64), 1.0 / 8.0),
        ((2, 4, 5, 16), (2, 2, 5, 16), 0.25),
        ((1, 2, 3, 8), (1, 1, 7, 8), 0.5),
    ]
    for qs, ks, scale in cases:
        Q = r.standard_normal(qs)
        K = r.standard_normal(ks)
        V = r.standard_normal(ks)
        for causal in (False, True):
            got = A.attention(Q, K, V, scale, causal)
            assert got.shape == qs, "output shape differs from Q's"
            want = np.array(_brute_force(Q.tolist(), K.tolist(), V.tolist(), scale, causal))
            _close(got, want, 1e-12, f"brute force {qs} causal={causal}")


def pin_identity_values_give_weights():
    """With V = I (T_kv == D) the output rows are the softmax weights, which
    must equal scipy's softmax of brute-force scores with -inf on masked keys."""
    r = _rng(8)
    T = 12
    Q = r.standard_normal((1, 1, T, T))
    K = r.standard_normal((1, 1, T, T))
    V = np.eye(T)[None, None]
    scale = 0.3
    logits = np.empty((T, T))
    for i in range(T):
        for j in range(T):
            logits[i, j] = scale * math.fsum(Q[0, 0, i, d] * K[0, 0, j, d] for d in range(T))
    for causal in (False, True):
        z = logits.copy()
        if causal:
            z[np.triu_indices(T, 1)] = -np.inf
        want = special.softmax(z, axis=1)
        got = A.attention(Q, K, V, scale, causal)[0, 0]
        _close(got, want, 1e-13, f"V = I gives the weights (causal={causal})")


# --- the 4x4 pattern printed on the page ---------------------------------------
def load_causal_golden():
    rows = [ln.split() for ln in (GOLDEN / "causal_mask_4x4.txt").read_text().splitlines()
            if ln.strip() and not ln.startswith("#")]
    return np.array([[int(x) for x in row] for row in rows], dtype=bool)


def pin_causal_pattern_4x4():
    """The oracle's keep-mask for seq_len 4 is the page's 4x4 example, and its
    weights are zero exactly where the example puts -inf."""
    want = load_causal_golden()
    got = A.visible(np.arange(4), 4, 4, True)
    assert np.array_equal(got, want), f"causal mask\n{got.astype(int)}\n!= page\n{want.astype(int)}"
    r = _rng(9)
    q, k, v = (r.standard_normal((4, 8)) for _ in range(3))
    _, p = A.attention_head(q, k, v, 0.5, True, return_p=True)
    assert np.array_equal(p > 0, want), "weights are not zero exactly at masked positions"


# --- invariances -----------------------------------------------------------------
def pin_shift_invariance():
    """Adding one vector u to every key adds q.u to all scores of a row, which
    the softmax ignores (AIInfraGuide page, section 7.2)."""
    r = _rng(10)
    Q = r.standard_normal((1, 2, 8, 16))
    K = r.standard_normal((1, 2, 8, 16))
    V = r.standard_normal((1, 2, 8, 16))
    u = 3.0 * r.standard_normal(16)
    for causal in (False, True):
        a = A.attention(Q, K, V, 0.5, causal)
        b = A.attention(Q, K + u, V, 0.5, causal)
        _close(a, b, 1e-10, f"shift invariance (causal={causal})")


def pin_large_logits():
    """Scores far beyond exp's range must not overflow (the max-subtraction of
    AIInfraGuide section 7.2); a huge scale turns the softmax into a one-hot
    at the row's largest score."""
    r = _rng(11)
    T, D = 10, 8
    Q = r.standard_normal((1, 1, T, D))
    K = r.standard_normal((1, 1, T, D))
    V = r.standard_normal((1, 1, T, D))
    raw = Q[0, 0] @ K[0, 0].T
    gaps = np.sort(raw, axis=1)
    assert np.all(gaps[:, -1] - gaps[:, -2] > 1e-3), "test input needs distinct maxima"
    O = A.attention(Q, K, V, 1e6, False)
    want = V[0, 0, np.argmax(raw, axis=1)]
    _close(O[0, 0], want, 1e-12, "one-hot at huge scale")


def pin_key_permutation():
    """Non-causal: permuting keys and values together leaves O unchanged;
    permuting queries permutes the rows of O."""
    r = _rng(12)
    Q = r.standard_normal((1, 1, 7, 8))
    K = r.standard_normal((1, 1, 9, 8))
    V = r.standard_normal((1, 1, 9, 8))
    base = A.attention(Q, K, V, 0.4, False)
    pk = r.permutation(9)
    _close(A.attention(Q, K[:, :, pk], V[:, :, pk], 0.4, False), base, 1e-13, "key permutation")
    pq = r.permutation(7)
    _close(A.attention(Q[:, :, pq], K, V, 0.4, False), base[:, :, pq], 1e-13, "query permutation")


def pin_linear_in_values():
    """O is linear in V for fixed Q, K."""
    r = _rng(13)
    Q = r.standard_normal((1, 2, 6, 8))
    K = r.standard_normal((1, 1, 6, 8))
    V1 = r.standard_normal((1, 1, 6, 8))
    V2 = r.standard_normal((1, 1, 6, 8))
    for causal in (False, True):
        lhs = A.attention(Q, K, 2.0 * V1 - 3.0 * V2, 0.3, causal)
        rhs = 2.0 * A.attention(Q, K, V1, 0.3, causal) - 3.0 * A.attention(Q, K, V2, 0.3, causal)
        _close(lhs, rhs, 1e-12, "linearity in V")


# --- a second formulation: online softmax + block merge ---------------------------
def _online_tiles(q, k, v, scale, causal, tile_sizes):
    """Independent formulation: per query row, walk the keys in tiles; keep the
    running maximum m, the rescaled exponential sum l and the output O, and
    merge each tile's (m, l, O) into them by the rules of AIInfraGuide
    sections 7.3 (the online recurrence) and 12.3 (merging two blocks)."""
    T_q, T_kv = q.shape[0], k.shape[0]
    off = T_kv - T_q
    out = np.empty((T_q, v.shape[1]))
    for i in range(T_q):
        m, l, o = -math.inf, 0.0, np.zeros(v.shape[1])
        j0 = 0
        t = 0
        while j0 < T_kv:
            j1 = min(T_kv, j0 + tile_sizes[t % len(tile_sizes)])
            t += 1
            vis = [j for j in range(j0, j1) if (not causal) or j <= i + off]
            j0 = j1
            if not vis:
                continue
            z = [scale * float(q[i] @ k[j]) for j in vis]
            m2 = max(z)
            w = [math.exp(x - m2) for x in z]
            l2 = math.fsum(w)
            o2 = sum(wj * v[j] for wj, j in zip(w, vis)) / l2  # block-local output
            m_new = max(m, m2)
            a1 = 0.0 if m == -math.inf else math.exp(m - m_new)
            a2 = math.exp(m2 - m_new)
            l_new = l * a1 + l2 * a2
            o = (o * l * a1 + o2 * l2 * a2) / l_new
            m, l = m_new, l_new
        out[i] = o
    return out


def pin_online_merge_equals_three_pass():
    """The tiled online-softmax formulation equals the oracle's three-pass
    result; the pages state the two are mathematically identical."""
    r = _rng(14)
    for causal, T_q, T_kv, tiles in [(False, 6, 17, [4]), (True, 13, 13, [3, 5]),
                                     (True, 4, 11, [2, 7, 1]), (False, 5, 5, [1])]:
        q = r.standard_normal((T_q, 8))
        k = 2.0 * r.standard_normal((T_kv, 8))
        v = r.standard_normal((T_kv, 8))
        got = A.attention_head(q, k, v, 0.7, causal)
        want = _online_tiles(q, k, v, 0.7, causal, tiles)
        _close(got, want, 1e-12, f"online merge (causal={causal}, tiles={tiles})")


def pin_window_one_sees_only_itself():
    """A window of one key: each row's softmax has a single term, so the
    output row is exactly the value row at the query's own position."""
    r = _rng(15)
    for T_q, T_kv in [(9, 9), (4, 11)]:
        q, k, v = (r.standard_normal((n, 6)) for n in (T_q, T_kv, T_kv))
        o = A.attention_head(q, k, v, 0.9, True, window=1)
        off = T_kv - T_q
        assert np.array_equal(o, v[np.arange(T_q) + off]), "window=1 must pick V[i + off]"


def pin_window_equals_truncated_keys():
    """Sliding window = plain (non-causal) attention of each row over the keys
    inside its window, taken as a separate problem; a window covering every
    key is plain causal attention."""
    r = _rng(16)
    T_q, T_kv, D, W = 10, 14, 5, 4
    q, k, v = (r.standard_normal((n, D)) for n in (T_q, T_kv, T_kv))
    o = A.attention_head(q, k, v, 0.6, True, window=W)
    off = T_kv - T_q
    for i in range(T_q):
        p = i + off
        lo = max(0, p - W + 1)
        want = A.attention_head(q[i:i + 1], k[lo:p + 1], v[lo:p + 1], 0.6, False)
        _close(o[i:i + 1], want, 1e-13, f"window row {i}")
    _close(A.attention_head(q, k, v, 0.6, True, window=T_kv), A.attention_head(q, k, v, 0.6, True),
           0.0, "window >= T_kv")


def pin_chunk_is_tail_of_full_prefill():
    """Chunked prefill: T_q queries placed at the end of T_kv keys (bottom-
    right causal) give exactly the last T_q rows of the full causal prefill
    whose queries are all T_kv positions."""
    r = _rng(17)
    T_kv, T_q, D = 12, 5, 4
    q_full = r.standard_normal((T_kv, D))
    k, v = r.standard_normal((T_kv, D)), r.standard_normal((T_kv, D))
    full = A.attention_head(q_full, k, v, 0.8, True)
    chunk = A.attention_head(q_full[-T_q:], k, v, 0.8, True)
    _close(chunk, full[-T_q:], 1e-13, "chunk vs full prefill")
    win_full = A.attention_head(q_full, k, v, 0.8, True, window=3)
    win_chunk = A.attention_head(q_full[-T_q:], k, v, 0.8, True, window=3)
    _close(win_chunk, win_full[-T_q:], 1e-13, "windowed chunk vs full")


def pin_varlen_is_independent_sequences():
    """A packed batch is B independent problems: with equal lengths it is the
    dense [B][H][T][D] result transposed to token-major, and a sequence's
    output does not depend on its neighbours."""
    r = _rng(18)
    B, H_q, H_kv, T, D = 3, 4, 2, 7, 5
    Q = r.standard_normal((B, H_q, T, D))
    K = r.standard_normal((B, H_kv, T, D))
    V = r.standard_normal((B, H_kv, T, D))
    dense = A.attention(Q, K, V, 0.5, True)
    packed = lambda X: X.transpose(0, 2, 1, 3).reshape(B * T, X.shape[1], D)
    cu = np.arange(B + 1) * T
    got = A.attention_varlen(packed(Q), packed(K), packed(V), cu, cu, 0.5, True)
    _close(got, packed(dense), 1e-13, "varlen vs dense")
    # ragged: sequence 1 alone equals its slice of the packed result
    cu_q, cu_k = np.array([0, 2, 7, 9]), np.array([0, 5, 9, 14])
    q = r.standard_normal((9, H_q, D))
    k = r.standard_normal((14, H_kv, D))
    v = r.standard_normal((14, H_kv, D))
    allo = A.attention_varlen(q, k, v, cu_q, cu_k, 0.5, True)
    one = A.attention_varlen(q[2:7], k[5:9], v[5:9], np.array([0, 5]), np.array([0, 4]), 0.5, True)
    _close(allo[2:7], one, 1e-13, "sequence independent of neighbours")
    # rows before the first key (T_q > T_kv) and empty key ranges give 0
    assert np.all(allo[2] == 0), "causal row with no visible key must be 0"
    empty = A.attention_varlen(q[:2], k[:0], v[:0], np.array([0, 2]), np.array([0, 0]), 0.5, False)
    assert np.all(empty == 0)


ALL_PINS = [
    pin_rows_sum_to_one,
    pin_causal_row0_is_v0,
    pin_zero_query_gives_mean,
    pin_gqa_is_repeated_mha,
    pin_single_key,
    pin_two_keys_sigmoid,
    pin_brute_force_worked_shape,
    pin_identity_values_give_weights,
    pin_causal_pattern_4x4,
    pin_shift_invariance,
    pin_large_logits,
    pin_key_permutation,
    pin_linear_in_values,
    pin_online_merge_equals_three_pass,
    pin_window_one_sees_only_itself,
    pin_window_equals_truncated_keys,
    pin_chunk_is_tail_of_full_prefill,
    pin_varlen_is_independent_sequences,
]
