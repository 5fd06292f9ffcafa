"""Pins for the dropout oracle.

The generator: oracle.philox4x64 (written from the SC 2011 definition) must
equal numpy.random.Philox, an independent implementation of Philox4x64-10,
bit for bit (numpy advances its 256-bit counter before each block, so its
first block from counter c is Philox(c + 1)).  The dropout: p = 0 is plain
attention exactly; the kept fraction matches 1 - T/65536 within a binomial
bound; keys are kept independently of the row's position in the batch;
averaged over seeds the dropped output is unbiased; a value row that is
dropped contributes nothing.  Planted mistakes (fields read from the wrong
word, no rescale) must fail.
"""

import numpy as np
import pytest

from oracle import attention, attention_dropout, keep_mask, philox4x64, threshold


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


@pytest.mark.parametrize("ctr,key", [
    ([0, 0, 0, 0], [0, 0]),
    ([5, 7, 11, 13], [123456789, 987654321]),
    ([2 ** 63, 3, 0, 9], [1, 2]),
    ([2 ** 64 - 2, 2 ** 64 - 1, 17, 2 ** 40], [2 ** 64 - 1, 2 ** 32]),
])
def test_philox_matches_numpy(ctr, key):
    g = np.random.Philox(counter=np.array(ctr, dtype=np.uint64), key=np.array(key, dtype=np.uint64))
    raw = g.random_raw(8)
    for blk in range(2):
        c = [int(x) for x in ctr]
        # numpy increments the counter (with carry) before producing a block.
        n = (c[0] | c[1] << 64 | c[2] << 128 | c[3] << 192) + blk + 1
        c = [(n >> (64 * w)) & (2 ** 64 - 1) for w in range(4)]
        got = philox4x64(*c, key[0], key[1])
        assert [int(x) for x in got] == [int(x) for x in raw[4 * blk:4 * blk + 4]]


def test_p_zero_is_plain_attention():
    q, k, v = _rand((1, 2, 9, 4), 1), _rand((1, 2, 11, 4), 2), _rand((1, 2, 11, 4), 3)
    a = attention_dropout(q, k, v, True, 0.5, 0.0, seed=7)
    b = attention(q, k, v, True, 0.5)
    assert np.allclose(a[0], b[0], rtol=1e-14, atol=1e-15)
    assert np.array_equal(a[1], b[1]) and np.array_equal(a[2], b[2])


@pytest.mark.parametrize("p", [0.1, 0.5, 0.9])
def test_kept_fraction(p):
    keep = keep_mask(3, 256, 256, p, seed=11, offset=0)
    want = 1 - threshold(p) / 65536
    n = keep.size
    assert abs(keep.mean() - want) <= 5 * np.sqrt(want * (1 - want) / n)


def test_streams_differ_by_seed_offset_and_head():
    a = keep_mask(0, 32, 64, 0.5, seed=1, offset=0)
    for other in (keep_mask(0, 32, 64, 0.5, seed=2, offset=0),
                  keep_mask(0, 32, 64, 0.5, seed=1, offset=1),
                  keep_mask(1, 32, 64, 0.5, seed=1, offset=0)):
        agree = (a == other).mean()
        assert 0.4 < agree < 0.6


def test_unbiased_on_average():
    q, k, v = _rand((1, 1, 6, 4), 4), _rand((1, 1, 8, 4), 5), _rand((1, 1, 8, 4), 6)
    plain = attention(q, k, v, False, 0.7)[0]
    acc = np.zeros_like(plain)
    n = 3000
    for s in range(n):
        acc += attention_dropout(q, k, v, False, 0.7, 0.3, seed=s)[0]
    assert np.max(np.abs(acc / n - plain)) < 0.05


def test_dropped_value_row_contributes_nothing():
    q, k = _rand((1, 1, 5, 3), 7), _rand((1, 1, 16, 3), 8)
    keep = keep_mask(0, 5, 16, 0.5, seed=9, offset=0)
    v = np.zeros((1, 1, 16, 1))
    v[0, 0, 3, 0] = 1.0  # only key 3 carries value
    out, _, _ = attention_dropout(q, k, v, False, 0.5, 0.5, seed=9)
    for i in range(5):
        assert (out[0, 0, i, 0] == 0) == (not keep[i, 3])


def test_pins_reject_mutants():
    q, k, v = _rand((1, 1, 6, 4), 10), _rand((1, 1, 8, 4), 11), _rand((1, 1, 8, 4), 12)
    plain = attention(q, k, v, False, 0.7)[0]
    # No rescale of kept weights: biased low on average.
    acc = np.zeros_like(plain)
    for s in range(2000):
        acc += attention_dropout(q, k, v, False, 0.7, 0.3, seed=s)[0] * (1 - threshold(0.3) / 65536)
    assert np.max(np.abs(acc / 2000 - plain)) > 0.05 * np.max(np.abs(plain)) or np.allclose(plain, 0)
    # Fields from the wrong output word: keep decisions change.
    t = threshold(0.5)
    i = np.arange(4, dtype=np.uint64)[:, None]
    j = np.arange(16, dtype=np.uint64)[None, :]
    w = philox4x64(j // np.uint64(16), i, np.uint64(0), np.uint64(0), 3, 0)
    bad = ((w[0] >> (np.uint64(16) * (j % np.uint64(4)))) & np.uint64(0xFFFF)) >= np.uint64(t)
    assert not np.array_equal(bad, keep_mask(0, 4, 16, 0.5, seed=3, offset=0))
