"""Pins of the QKV-projection oracle (``oracle.qkv_fp64``): scalar brute
force on a tiny shape (explicit loops over tokens, features and the reduction
index, with the head split written per element), one-hot weight rows that
copy chosen input columns into chosen (head, feature) slots, and linearity in
W.  Planted mistakes in the split are each caught."""
import numpy as np
import pytest

import oracle.qkv_fp64 as P


def pin_brute_force_tiny():
    rng = np.random.default_rng(21)
    B, T, dm, H_q, H_kv, D = 2, 3, 5, 2, 1, 2
    N = (H_q + 2 * H_kv) * D
    x = rng.standard_normal((B * T, dm))
    w = rng.standard_normal((N, dm))
    q, k, v = P.qkv_project(x, w, B, T, H_q, H_kv, D)
    for b in range(B):
        for t in range(T):
            for n in range(N):
                acc = 0.0
                for kk in range(dm):
                    acc += float(x[b * T + t, kk]) * float(w[n, kk])
                if n < H_q * D:
                    got = q[b, n // D, t, n % D]
                elif n < (H_q + H_kv) * D:
                    got = k[b, (n - H_q * D) // D, t, n % D]
                else:
                    got = v[b, (n - (H_q + H_kv) * D) // D, t, n % D]
                assert abs(got - acc) < 1e-12


def pin_one_hot_rows_copy_columns():
    rng = np.random.default_rng(22)
    B, T, dm, H_q, H_kv, D = 2, 4, 8, 2, 1, 4
    N = (H_q + 2 * H_kv) * D
    x = rng.standard_normal((B * T, dm))
    src = rng.integers(0, dm, N)               # output feature n copies input column src[n]
    w = np.zeros((N, dm))
    w[np.arange(N), src] = 1.0
    q, k, v = P.qkv_project(x, w, B, T, H_q, H_kv, D)
    # V of kv head 0, feature 3, token (b=1, t=2) is input column src[(H_q + H_kv) D + 3] of row 1*T + 2
    assert v[1, 0, 2, 3] == x[1 * T + 2, src[(H_q + H_kv) * D + 3]]
    assert q[0, 1, 3, 0] == x[3, src[1 * D + 0]]
    assert k[1, 0, 0, 2] == x[T, src[H_q * D + 2]]


def pin_linear_in_weights():
    rng = np.random.default_rng(23)
    x = rng.standard_normal((6, 8))
    w1, w2 = rng.standard_normal((16, 8)), rng.standard_normal((16, 8))
    a = P.qkv_project(x, w1 + 2 * w2, 2, 3, 2, 1, 4)
    b1, b2 = P.qkv_project(x, w1, 2, 3, 2, 1, 4), P.qkv_project(x, w2, 2, 3, 2, 1, 4)
    for i in range(3):
        assert np.max(np.abs(a[i] - (b1[i] + 2 * b2[i]))) < 1e-12


PINS = [pin_brute_force_tiny, pin_one_hot_rows_copy_columns, pin_linear_in_weights]


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_qkv_pin_holds(pin):
    pin()


def _split_kv_swapped(y, B, T, H_q, H_kv, D):
    q, k, v = _orig(y, B, T, H_q, H_kv, D)
    return q, v, k


def _split_no_transpose(y, B, T, H_q, H_kv, D):
    qn, kn = H_q * D, H_kv * D
    f = lambda blk, H: blk.reshape(B, H, T, D)   # treats rows as head-major
    return f(y[:, :qn], H_q), f(y[:, qn:qn + kn], H_kv), f(y[:, qn + kn:], H_kv)


_orig = P.split_heads


@pytest.mark.parametrize("mutant", [_split_kv_swapped, _split_no_transpose], ids=lambda f: f.__name__)
def test_planted_split_mistakes_are_caught(mutant, monkeypatch):
    monkeypatch.setattr(P, "split_heads", mutant)
    caught = 0
    for pin in PINS:
        try:
            pin()
        except AssertionError:
            caught += 1
    assert caught > 0
