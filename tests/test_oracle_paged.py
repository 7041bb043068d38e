"""Pins of the paged-cache decode oracle (``oracle.paged_fp64``).

The paged oracle is a gather followed by the already pinned attention oracle,
so its pins target the gather: equivalence with the contiguous oracle on the
same keys (any wrong page, row or kv-head index breaks it), invariance under
a permutation of the pool, a single key (the output is that key's value row
exactly), and the readings for empty sequences and out-of-pool block ids.
Each pin is also run against planted mistakes in the gather.
"""
import numpy as np
import pytest

import oracle.attention_fp64 as A
import oracle.paged_fp64 as P


def _paged_layout(K, V, page_size, rng, extra_pages=5):
    """Scatter contiguous K, V [B, H_kv, T, D] into shuffled pools; returns
    (k_pages, v_pages, block_table)."""
    B, H_kv, T, D = K.shape
    per_seq = -(-T // page_size)
    n_pages = B * per_seq + extra_pages
    perm = rng.permutation(n_pages)
    kp = rng.standard_normal((n_pages, H_kv, page_size, D))  # junk in unused rows/pages
    vp = rng.standard_normal((n_pages, H_kv, page_size, D))
    table = np.empty((B, per_seq), np.int64)
    for b in range(B):
        for p in range(per_seq):
            phys = perm[b * per_seq + p]
            table[b, p] = phys
            rows = slice(p * page_size, min(T, (p + 1) * page_size))
            n = rows.stop - rows.start
            kp[phys, :, :n] = K[b, :, rows]
            vp[phys, :, :n] = V[b, :, rows]
    return kp, vp, table


def _contiguous(q, K, V, lens, scale):
    B, H_q, D = q.shape
    H_kv = K.shape[1]
    out = np.zeros((B, H_q, D))
    for b in range(B):
        for h in range(H_q):
            g = A.kv_head_for(h, H_q, H_kv)
            L = lens[b]
            if L:
                out[b, h] = A.attention_head(q[b, h][None], K[b, g, :L], V[b, g, :L], scale, False)[0]
    return out


def pin_matches_contiguous_oracle():
    rng = np.random.default_rng(7)
    B, H_q, H_kv, T, D, ps = 3, 6, 2, 70, 8, 16
    q = rng.standard_normal((B, H_q, D))
    K = rng.standard_normal((B, H_kv, T, D))
    V = rng.standard_normal((B, H_kv, T, D))
    kp, vp, table = _paged_layout(K, V, ps, rng)
    lens = np.array([70, 33, 16])
    got = P.decode_paged(q, kp, vp, table, lens, 0.3)
    want = _contiguous(q, K, V, lens, 0.3)
    assert np.max(np.abs(got - want)) < 1e-12


def pin_pool_permutation_invariant():
    rng = np.random.default_rng(8)
    B, H_q, H_kv, T, D, ps = 2, 4, 4, 50, 4, 16
    q = rng.standard_normal((B, H_q, D))
    K = rng.standard_normal((B, H_kv, T, D))
    V = rng.standard_normal((B, H_kv, T, D))
    kp, vp, table = _paged_layout(K, V, ps, rng)
    lens = np.array([50, 41])
    a = P.decode_paged(q, kp, vp, table, lens, 0.5)
    perm = rng.permutation(kp.shape[0])          # physical page i moves to perm[i]
    kp2, vp2 = np.empty_like(kp), np.empty_like(vp)
    kp2[perm], vp2[perm] = kp, vp
    b = P.decode_paged(q, kp2, vp2, perm[table], lens, 0.5)
    assert np.max(np.abs(a - b)) < 1e-12


def pin_single_key_returns_its_value_row():
    rng = np.random.default_rng(9)
    B, H_q, H_kv, D, ps = 2, 4, 2, 8, 16
    kp = rng.standard_normal((6, H_kv, ps, D))
    vp = rng.standard_normal((6, H_kv, ps, D))
    table = np.array([[4, 1], [2, 0]])
    q = rng.standard_normal((B, H_q, D))
    out = P.decode_paged(q, kp, vp, table, np.array([1, 1]), 1.7)
    for b in range(B):
        for h in range(H_q):
            assert np.array_equal(out[b, h], vp[table[b, 0], h // 2, 0])


def pin_empty_and_clamped_lengths():
    rng = np.random.default_rng(10)
    kp = rng.standard_normal((4, 1, 16, 4))
    vp = rng.standard_normal((4, 1, 16, 4))
    q = rng.standard_normal((3, 2, 4))
    table = np.array([[0, 1], [2, 3], [1, 0]])
    out = P.decode_paged(q, kp, vp, table, np.array([0, -5, 999]), 1.0)
    assert np.all(out[0] == 0) and np.all(out[1] == 0)
    full = P.decode_paged(q, kp, vp, table, np.array([0, 0, 32]), 1.0)
    assert np.array_equal(out[2], full[2])  # 999 clamps to 2 pages x 16


def pin_out_of_pool_block_reads_zeros():
    rng = np.random.default_rng(11)
    kp = rng.standard_normal((3, 1, 16, 4))
    vp = rng.standard_normal((3, 1, 16, 4))
    q = rng.standard_normal((1, 1, 4))
    # every page outside the pool: all keys zero -> uniform weights over zero values
    out = P.decode_paged(q, kp, vp, np.array([[-1, 3]]), np.array([20]), 1.0)
    assert np.all(out == 0)
    # one zero page next to a real one: the zero keys score 0 and add exp(0 - m)
    # to the denominator; compare with an explicit zero page in the pool
    kz = np.concatenate([kp, np.zeros((1, 1, 16, 4))])
    vz = np.concatenate([vp, np.zeros((1, 1, 16, 4))])
    a = P.decode_paged(q, kp, vp, np.array([[1, 7]]), np.array([32]), 1.0)
    b = P.decode_paged(q, kz, vz, np.array([[1, 3]]), np.array([32]), 1.0)
    assert np.max(np.abs(a - b)) < 1e-15


PINS = [pin_matches_contiguous_oracle, pin_pool_permutation_invariant,
        pin_single_key_returns_its_value_row, pin_empty_and_clamped_lengths,
        pin_out_of_pool_block_reads_zeros]


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_paged_pin_holds(pin):
    pin()


def _mutant_row(pages, block_row, seq_len, page_size, kv_head):
    # wrong row within the page: (j + 1) % page_size
    j = np.arange(seq_len)
    page = np.asarray(block_row)[j // page_size]
    return np.asarray(pages[page, kv_head, (j + 1) % page_size], np.float64)


def _mutant_page(pages, block_row, seq_len, page_size, kv_head):
    # logical page used as the physical page (block table ignored)
    j = np.arange(seq_len)
    return np.asarray(pages[(j // page_size) % pages.shape[0], kv_head, j % page_size], np.float64)


def _mutant_head(pages, block_row, seq_len, page_size, kv_head):
    # kv head ignored (head 0 for every q head)
    j = np.arange(seq_len)
    page = np.asarray(block_row)[j // page_size]
    return np.asarray(pages[page, 0, j % page_size], np.float64)


@pytest.mark.parametrize("mutant", [_mutant_row, _mutant_page, _mutant_head],
                         ids=lambda f: f.__name__)
def test_planted_gather_mistakes_are_caught(mutant, monkeypatch):
    monkeypatch.setattr(P, "gather_sequence", mutant)
    with pytest.raises(AssertionError):
        pin_matches_contiguous_oracle()
