"""Plant plausible mistakes in the oracle (on the CPU) and check that the pins
catch every one of them.  Each mutant replaces one oracle function; the
pitfalls listed on the Ch. 11 page ("常见坑": wrong mask direction, scale,
mixed-up Q/K/V) are among them."""
import math

import numpy as np
import pytest

import oracle.attention_fp64 as A
import pins

_orig_visible = A.visible
_orig_scores = A.scores
_orig_softmax = A.softmax_rows
_orig_weighted = A.weighted_sum
_orig_kv_head = A.kv_head_for
_orig_head = A.attention_head


def _with_window(m, rows, T_q, T_kv, window):
    if window <= 0:
        return m
    pos = np.asarray(rows)[:, None] + (T_kv - T_q)
    return m & (np.arange(T_kv)[None, :] > pos - window)


def _mask_flipped(rows, T_q, T_kv, causal, window=0):
    m = _orig_visible(rows, T_q, T_kv, causal, window)
    if not causal:
        return m
    rows = np.asarray(rows)
    j = np.arange(T_kv)
    return _with_window(j[None, :] >= rows[:, None] + (T_kv - T_q), rows, T_q, T_kv, window)


def _mask_strict(rows, T_q, T_kv, causal, window=0):
    if not causal:
        return _orig_visible(rows, T_q, T_kv, causal, window)
    rows = np.asarray(rows)
    j = np.arange(T_kv)
    return _with_window(j[None, :] < rows[:, None] + (T_kv - T_q), rows, T_q, T_kv, window)


def _mask_top_left(rows, T_q, T_kv, causal, window=0):
    if not causal:
        return _orig_visible(rows, T_q, T_kv, causal, window)
    rows = np.asarray(rows)
    j = np.arange(T_kv)
    return _with_window(j[None, :] <= rows[:, None], rows, T_q, T_kv, window)


def _window_one_too_wide(rows, T_q, T_kv, causal, window=0):
    m = _orig_visible(rows, T_q, T_kv, causal, 0)
    if not causal or window <= 0:
        return m
    pos = np.asarray(rows)[:, None] + (T_kv - T_q)
    return m & (np.arange(T_kv)[None, :] >= pos - window)


def _window_ignored(rows, T_q, T_kv, causal, window=0):
    return _orig_visible(rows, T_q, T_kv, causal, 0)


def _kv_head_tiled(h_q, H_q, H_kv):
    return h_q % H_kv


def _softmax_no_max(s, keep):
    e = np.where(keep, np.exp(s), 0.0)
    return e / e.sum(axis=1, keepdims=True)


def _softmax_unnormalised(s, keep):
    z = np.where(keep, s, -np.inf)
    return np.exp(z - z.max(axis=1, keepdims=True))


def _softmax_over_columns(s, keep):
    z = np.where(keep, s, -np.inf)
    m = np.max(np.where(np.isfinite(z), z, -1e300), axis=0, keepdims=True)
    e = np.where(keep, np.exp(z - m), 0.0)
    tot = e.sum(axis=0, keepdims=True)
    return e / np.where(tot > 0, tot, 1.0)


def _scores_scale_squared(q_rows, k, scale):
    return _orig_scores(q_rows, k, scale * scale)


def _scores_unscaled(q_rows, k, scale):
    return _orig_scores(q_rows, k, 1.0)


def _scores_transposed(q_rows, k, scale):
    s = _orig_scores(q_rows, k, scale)
    if s.shape[0] == s.shape[1]:
        return s.T.copy()
    return s[:, ::-1].copy()


def _head_swapped_kv(q, k, v, scale, causal, rows=None, return_p=False, window=0):
    return _orig_head(q, v, k, scale, causal, rows, return_p, window)


def _weighted_sum_first_key_dropped(p, v):
    p = p.copy()
    p[:, 0] = 0.0
    return _orig_weighted(p, v)


MUTANTS = {
    "mask_direction_flipped": ("visible", _mask_flipped),
    "mask_excludes_diagonal": ("visible", _mask_strict),
    "causal_top_left_aligned": ("visible", _mask_top_left),
    "window_one_key_too_wide": ("visible", _window_one_too_wide),
    "window_ignored": ("visible", _window_ignored),
    "gqa_heads_tiled_not_grouped": ("kv_head_for", _kv_head_tiled),
    "softmax_without_max_subtraction": ("softmax_rows", _softmax_no_max),
    "softmax_not_normalised": ("softmax_rows", _softmax_unnormalised),
    "softmax_over_wrong_axis": ("softmax_rows", _softmax_over_columns),
    "scale_applied_twice": ("scores", _scores_scale_squared),
    "scale_dropped": ("scores", _scores_unscaled),
    "scores_transposed": ("scores", _scores_transposed),
    "k_and_v_swapped": ("attention_head", _head_swapped_kv),
    "first_key_dropped": ("weighted_sum", _weighted_sum_first_key_dropped),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(A, attr, fn)
    caught = []
    import warnings
    with warnings.catch_warnings():
        warnings.simplefilter("ignore")
        for pin in pins.ALL_PINS:
            try:
                pin()
            except (AssertionError, ValueError, FloatingPointError, IndexError):
                caught.append(pin.__name__)
    assert caught, f"no pin caught the planted mistake {name!r}"
