"""Pins for the sliding-window rule and the paged-cache oracle.

Independent of the oracle's arithmetic: closed forms (a window of one key
returns that key's value row exactly; with Q = 0 the row sum l counts the
visible keys, an integer), a two-key window against 50-digit mpmath, the
window's limits (W >= Nk is plain causal attention), exact equality of the
page gather with the contiguous keys under shuffled and shared page tables,
and the grouped-head mapping against explicitly repeated K/V.  Planted
mistakes (an off-by-one window, a wrong head mapping, a wrong page offset)
must each fail.
"""

import mpmath
import numpy as np
import pytest

import oracle
from oracle import attention_paged, attention_rows, gather_pages, visible_mask


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


@pytest.mark.parametrize("nq,nk", [(7, 7), (3, 9), (9, 4)])
def test_window_one_returns_the_diagonal_value(nq, nk):
    q, k, v = _rand((nq, 5), 1), _rand((nk, 5), 2), _rand((nk, 5), 3)
    out, m, l = attention_rows(q, k, v, True, 0.4, window=1)
    for i in range(nq):
        j = i + nk - nq
        if j < 0:
            assert np.all(out[i] == 0) and l[i] == 0 and m[i] == -np.inf
        else:
            assert np.array_equal(out[i], v[j]) and l[i] == 1.0


@pytest.mark.parametrize("window", [1, 2, 3, 5, 100])
def test_window_counts_visible_keys(window):
    # Q = 0: every visible score is 0, so l is the count of visible keys.
    nq, nk = 6, 10
    _, _, l = attention_rows(np.zeros((nq, 4)), _rand((nk, 4), 4), _rand((nk, 4), 5), True, 1.0,
                             window=window)
    for i in range(nq):
        diag = i + nk - nq
        assert l[i] == min(window, diag + 1)


def test_wide_window_is_causal():
    q, k, v = _rand((8, 4), 6), _rand((11, 4), 7), _rand((11, 4), 8)
    a = attention_rows(q, k, v, True, 0.5, window=11)
    b = attention_rows(q, k, v, True, 0.5)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def test_two_key_window_against_mpmath():
    mpmath.mp.dps = 50
    q, k, v = _rand((4, 3), 9), _rand((6, 3), 10), _rand((6, 3), 11)
    out, _, _ = attention_rows(q, k, v, True, 0.7, window=2)
    for i in range(4):
        diag = i + 2
        js = [diag - 1, diag]
        s = [mpmath.mpf(0.7) * mpmath.fsum(mpmath.mpf(q[i, d]) * mpmath.mpf(k[j, d])
                                            for d in range(3)) for j in js]
        w = [mpmath.exp(x) for x in s]
        for d in range(3):
            ref = (w[0] * mpmath.mpf(v[js[0], d]) + w[1] * mpmath.mpf(v[js[1], d])) / (w[0] + w[1])
            assert abs(out[i, d] - float(ref)) <= 1e-14


def test_window_needs_causal():
    with pytest.raises(ValueError):
        visible_mask(4, 4, False, window=2)


def _paged_layout(k, v, page_size, seed, spare=3):
    """Scatter per-sequence K/V [B, Hkv, N, D] into shuffled pages."""
    b_, hkv, n, d = k.shape
    npp = (n + page_size - 1) // page_size
    total = b_ * npp + spare
    perm = np.random.default_rng(seed).permutation(total)
    kc = _rand((total, hkv, page_size, d), seed + 1)  # unused slots hold junk
    vc = _rand((total, hkv, page_size, d), seed + 2)
    table = np.zeros((b_, npp), dtype=np.int64)
    for b in range(b_):
        for p in range(npp):
            page = perm[b * npp + p]
            table[b, p] = page
            rows = slice(p * page_size, min(n, (p + 1) * page_size))
            cnt = rows.stop - rows.start
            kc[page, :, :cnt] = k[b, :, rows]
            vc[page, :, :cnt] = v[b, :, rows]
    return kc, vc, table


def test_gather_reproduces_contiguous_keys():
    k = _rand((2, 3, 37, 4), 12)
    kc, _, table = _paged_layout(k, k, 8, seed=13)
    for b in range(2):
        for h in range(3):
            for n in (0, 1, 8, 9, 37):
                assert np.array_equal(gather_pages(kc, table[b], h, n, 8), k[b, h, :n])


def test_shared_pages():
    # Two sequences that share their first page (a common prefix).
    kc = _rand((4, 1, 4, 2), 14)
    table = np.array([[2, 0], [2, 3]])
    a = gather_pages(kc, table[0], 0, 6, 4)
    b = gather_pages(kc, table[1], 0, 7, 4)
    assert np.array_equal(a[:4], b[:4]) and np.array_equal(a[:4], kc[2, 0])
    assert np.array_equal(b[4:], kc[3, 0, :3])


@pytest.mark.parametrize("causal,window", [(False, 0), (True, 0), (True, 5)])
def test_paged_equals_contiguous_with_repeated_heads(causal, window):
    b_, h_, hkv, nq, n, d = 2, 6, 2, 3, 29, 8
    q = _rand((b_, h_, nq, d), 15)
    k = _rand((b_, hkv, n, d), 16)
    v = _rand((b_, hkv, n, d), 17)
    kc, vc, table = _paged_layout(k, v, 4, seed=18)
    lens = np.array([29, 17])
    got, gm, gl = attention_paged(q, kc, vc, table, lens, causal, 0.3, window=window)
    for b in range(b_):
        for h in range(h_):
            hk = h // (h_ // hkv)
            want = attention_rows(q[b, h], k[b, hk, :lens[b]], v[b, hk, :lens[b]], causal, 0.3,
                                  window=window)
            assert np.array_equal(got[b, h], want[0])
            assert np.array_equal(gm[b, h], want[1]) and np.array_equal(gl[b, h], want[2])


def test_empty_sequence():
    q = _rand((1, 2, 2, 4), 19)
    kc = _rand((3, 1, 4, 4), 20)
    out, m, l = attention_paged(q, kc, kc, np.array([[1]]), np.array([0]), True, 0.5)
    assert np.all(out == 0) and np.all(m == -np.inf) and np.all(l == 0)


def test_pins_reject_mutants():
    nq, nk = 6, 10
    z = np.zeros((nq, 4))
    kk, vv = _rand((nk, 4), 21), _rand((nk, 4), 22)
    # Off-by-one window (one key too many).
    diag = np.arange(nq)[:, None] + nk - nq
    j = np.arange(nk)[None, :]
    vis_bad = (j <= diag) & (j >= diag - 3)
    l_bad = vis_bad.sum(axis=1)
    _, _, l = attention_rows(z, kk, vv, True, 1.0, window=3)
    assert not np.array_equal(l, l_bad)
    # Head mapping h % Hkv instead of h // group.
    k = _rand((1, 2, 9, 4), 23)
    kc, vc, table = _paged_layout(k, k, 4, seed=24)
    q = _rand((1, 4, 2, 4), 25)
    got, _, _ = attention_paged(q, kc, vc, table, np.array([9]), False, 0.5)
    bad = attention_rows(q[0, 1], k[0, 1 % 2], k[0, 1 % 2], False, 0.5)[0]
    assert not np.allclose(got[0, 1], bad)
    # Page offset taken from the wrong page size.
    assert not np.array_equal(gather_pages(kc, table[0], 0, 6, 2), k[0, 0, :6])


def test_oracle_package_exports():
    assert oracle.attention_paged is attention_paged
