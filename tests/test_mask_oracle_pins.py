"""Pins for the oracle's arbitrary mask and its window on the batched path.

Independent of its arithmetic: an all-true mask changes nothing (bitwise); a
mask with one true key per row returns that key's value row exactly with
l = 1; with Q = 0, l counts the keys that the mask, the causal rule and
the window all leave visible (integer closed form); the causal pattern given
as a mask reproduces causal attention bitwise; an all-false row gives
out = 0 and the empty state.  Planted mistakes (the mask ignored, the mask
transposed) must fail.
"""

import numpy as np
import pytest

from oracle import attention, attention_rows


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def test_all_true_mask_changes_nothing():
    q, k, v = _rand((2, 3, 9, 4), 1), _rand((2, 3, 11, 4), 2), _rand((2, 3, 11, 4), 3)
    a = attention(q, k, v, True, 0.5)
    b = attention(q, k, v, True, 0.5, mask=np.ones((9, 11), dtype=bool))
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def test_one_key_per_row():
    nq, nk = 7, 10
    q, k, v = _rand((nq, 4), 4), _rand((nk, 4), 5), _rand((nk, 4), 6)
    pick = np.random.default_rng(7).integers(0, nk, size=nq)
    mask = np.zeros((nq, nk), dtype=bool)
    mask[np.arange(nq), pick] = True
    out, _, l = attention_rows(q, k, v, False, 0.3, mask=mask)
    for i in range(nq):
        assert np.array_equal(out[i], v[pick[i]]) and l[i] == 1.0


@pytest.mark.parametrize("causal,window", [(False, 0), (True, 0), (True, 3)])
def test_zero_queries_count_mask_causal_and_window(causal, window):
    nq, nk = 6, 9
    mask = np.random.default_rng(8).random((nq, nk)) < 0.5
    _, _, l = attention_rows(np.zeros((nq, 3)), _rand((nk, 3), 9), _rand((nk, 3), 10), causal,
                             1.0, window=window, mask=mask)
    for i in range(nq):
        diag = i + nk - nq
        count = 0
        for j in range(nk):
            ok = mask[i, j] and (not causal or j <= diag) and (not window or j > diag - window)
            count += ok
        assert l[i] == count


def test_causal_pattern_as_mask_is_causal():
    nq, nk = 8, 12
    q, k, v = _rand((1, 2, nq, 5), 11), _rand((1, 2, nk, 5), 12), _rand((1, 2, nk, 5), 13)
    j = np.arange(nk)[None, :]
    i = np.arange(nq)[:, None]
    mask = j <= i + nk - nq
    a = attention(q, k, v, True, 0.7)
    b = attention(q, k, v, False, 0.7, mask=mask)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def test_all_false_row():
    mask = np.ones((3, 5), dtype=bool)
    mask[1] = False
    out, m, l = attention_rows(_rand((3, 2), 14), _rand((5, 2), 15), _rand((5, 2), 16), False, 1.0,
                               mask=mask)
    assert np.all(out[1] == 0) and m[1] == -np.inf and l[1] == 0


def test_pins_reject_mutants():
    nq, nk = 5, 5
    mask = np.random.default_rng(17).random((nq, nk)) < 0.5
    z = np.zeros((nq, 2))
    kk, vv = _rand((nk, 2), 18), _rand((nk, 2), 19)
    _, _, l = attention_rows(z, kk, vv, False, 1.0, mask=mask)
    assert not np.array_equal(l, np.full(nq, float(nk)))       # mask ignored
    assert not np.array_equal(l, mask.T.sum(axis=1).astype(float))  # mask transposed
    assert np.array_equal(l, mask.sum(axis=1).astype(float))
