"""Pins for the packed variable-length attention oracle.

Independent of its arithmetic: equal lengths reduce to the batched oracle on
the transposed layout (pins the packing and head indexing); with Q = 0 the
row sum l counts each row's visible keys, with causal keys aligned to the
end of each sequence's own query block (an integer closed form); sequences
are independent (changing one sequence's keys leaves every other sequence's
output unchanged); empty sequences give nothing.  Planted mistakes (keys
aligned to the packed block instead of the sequence, a wrong head mapping)
must fail.
"""

import numpy as np
import pytest

from oracle import attention, attention_varlen


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _cu(lens):
    return np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)


@pytest.mark.parametrize("causal", [False, True])
def test_equal_lengths_reduce_to_batched(causal):
    b, h, hkv, n, d = 3, 4, 2, 9, 5
    qb = _rand((b, h, n, d), 1)
    kb = _rand((b, hkv, n, d), 2)
    vb = _rand((b, hkv, n, d), 3)
    g = h // hkv
    want, wm, wl = attention(qb, np.repeat(kb, g, axis=1), np.repeat(vb, g, axis=1), causal, 0.4)
    q = qb.transpose(0, 2, 1, 3).reshape(b * n, h, d)
    k = kb.transpose(0, 2, 1, 3).reshape(b * n, hkv, d)
    v = vb.transpose(0, 2, 1, 3).reshape(b * n, hkv, d)
    cu = _cu([n] * b)
    out, m, l = attention_varlen(q, k, v, cu, cu, causal, 0.4)
    assert np.array_equal(out, want.transpose(0, 2, 1, 3).reshape(b * n, h, d))
    assert np.array_equal(m, wm.transpose(1, 0, 2).reshape(h, b * n))
    assert np.array_equal(l, wl.transpose(1, 0, 2).reshape(h, b * n))


def test_zero_queries_count_visible_keys_per_sequence():
    lq, lk = [4, 0, 7, 3], [6, 2, 3, 3]
    cu_q, cu_k = _cu(lq), _cu(lk)
    q = np.zeros((sum(lq), 2, 3))
    k, v = _rand((sum(lk), 2, 3), 4), _rand((sum(lk), 2, 3), 5)
    _, _, l = attention_varlen(q, k, v, cu_q, cu_k, True, 1.0)
    for b in range(4):
        for i in range(lq[b]):
            want = min(lk[b], max(0, i + lk[b] - lq[b] + 1))
            assert np.all(l[:, cu_q[b] + i] == want)


def test_sequences_are_independent():
    lq, lk = [5, 8, 3], [6, 8, 9]
    cu_q, cu_k = _cu(lq), _cu(lk)
    q = _rand((16, 2, 4), 6)
    k, v = _rand((23, 2, 4), 7), _rand((23, 2, 4), 8)
    a, _, _ = attention_varlen(q, k, v, cu_q, cu_k, False, 0.5)
    k2, v2 = k.copy(), v.copy()
    k2[6:14] += 3.0  # sequence 1's keys only
    v2[6:14] -= 1.0
    c, _, _ = attention_varlen(q, k2, v2, cu_q, cu_k, False, 0.5)
    assert np.array_equal(a[:5], c[:5]) and np.array_equal(a[13:], c[13:])
    assert not np.allclose(a[5:13], c[5:13])


def test_empty_sequences():
    cu = _cu([0, 3, 0])
    q, k = _rand((3, 1, 2), 9), _rand((3, 1, 2), 10)
    out, m, l = attention_varlen(q, k, k, cu, cu, True, 1.0)
    assert out.shape == (3, 1, 2) and np.all(np.isfinite(out)) and np.all(l > 0)


def test_pins_reject_mutants():
    # Causal keys aligned to the packed block instead of each sequence.
    lq, lk = [3, 5], [6, 5]
    cu_q, cu_k = _cu(lq), _cu(lk)
    z = np.zeros((8, 1, 2))
    k = _rand((11, 1, 2), 11)
    _, _, l = attention_varlen(z, k, k, cu_q, cu_k, True, 1.0)
    bad = np.array([min(11, i + 11 - 8 + 1) for i in range(8)], dtype=float)
    assert not np.array_equal(l[0], bad)
    # Head mapping h % Hkv instead of h // group.
    q = _rand((4, 4, 3), 12)
    kk, vv = _rand((4, 2, 3), 13), _rand((4, 2, 3), 14)
    cu = _cu([4])
    out, _, _ = attention_varlen(q, kk, vv, cu, cu, False, 0.5)
    qb = q.transpose(1, 0, 2)[None]
    bad_k = kk.transpose(1, 0, 2)[[0, 1, 0, 1]][None]
    bad_v = vv.transpose(1, 0, 2)[[0, 1, 0, 1]][None]
    bad_out, _, _ = attention(qb, bad_k, bad_v, False, 0.5)
    assert not np.allclose(out.transpose(1, 0, 2), bad_out[0])
