"""Pins for the FP64 row-softmax oracle and its split (A2) model.

Independent of the oracle's own arithmetic: the scratch size the answer-key
page prints (tests/golden/worked_examples.json, item A2), closed forms,
invariants (rows sum to one, shift and permutation behaviour), a library
routine (scipy.special.softmax) and 50-digit brute force.  Plausible
mistakes planted in copies of the row softmax must each fail at least one
pin, and the page's own mistake (chunk-local normalisation) must be caught.
"""

import json
import math
import os

import mpmath
import numpy as np
import pytest
import scipy.special

from oracle import num_chunks, scratch_bytes, softmax_rows, split_softmax_model

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_examples.json")


def test_a2_scratch_worked_example():
    g = json.load(open(GOLDEN))["a2_scratch"]
    assert num_chunks(g["N"], g["chunk"]) == g["expected_chunks"]
    assert scratch_bytes(g["M"], g["N"], g["chunk"]) == g["expected_scratch_bytes"]


# --------------------------------------------------------------------------
# Pins, written against an implementation argument so the mutants below can
# be run through the same checks.

def _pin_library(f):
    rng = np.random.default_rng(1)
    for shape in ((1, 1), (3, 7), (5, 300), (2, 4097)):
        x = rng.standard_normal(shape) * 3.0
        if not np.allclose(f(x), scipy.special.softmax(x, axis=1), rtol=1e-13, atol=0):
            return False
    return True


def _pin_closed_forms(f):
    ok = np.allclose(f(np.zeros((2, 5))), np.full((2, 5), 0.2), rtol=1e-15, atol=0)
    ok &= np.allclose(f(np.array([[0.0, math.log(3.0)]])), [[0.25, 0.75]], rtol=1e-15, atol=0)
    ok &= np.array_equal(f(np.array([[-3.5], [7.0]])), np.ones((2, 1)))
    # Rows are independent: how far another row sits changes nothing.
    a = f(np.array([[0.0, 1.0], [0.0, 50.0], [-2000.0, -1999.0]]))
    two = [1 / (1 + math.e), math.e / (1 + math.e)]
    ok &= np.allclose(a[0], two, rtol=1e-15, atol=0)
    ok &= np.allclose(a[2], two, rtol=1e-15, atol=0)
    return bool(ok)


def _pin_invariants(f):
    rng = np.random.default_rng(2)
    x = rng.standard_normal((4, 33))
    y = f(x)
    ok = np.all(np.isfinite(y)) and np.allclose(y.sum(axis=1), 1.0, rtol=0, atol=1e-14)
    # Shift invariance, including a shift that overflows exp() without the max.
    ok &= np.allclose(f(x + 1000.0), y, rtol=1e-12, atol=0)
    ok &= np.allclose(f(x - 1000.0), y, rtol=1e-12, atol=0)
    perm = rng.permutation(33)
    ok &= np.allclose(f(x[:, perm]), y[:, perm], rtol=1e-15, atol=0)
    # Order: larger logits get larger probabilities.
    ok &= bool(np.all(np.argsort(f(x), axis=1) == np.argsort(x, axis=1)))
    return bool(ok)


def _pin_brute_force(f):
    mpmath.mp.dps = 50
    rng = np.random.default_rng(3)
    for n in (1, 2, 5, 9):
        x = rng.standard_normal((2, n)) * 4.0
        y = f(x)
        for r in range(2):
            den = mpmath.fsum(mpmath.exp(mpmath.mpf(float(v))) for v in x[r])
            for j in range(n):
                want = float(mpmath.exp(mpmath.mpf(float(x[r, j]))) / den)
                if abs(y[r, j] - want) > 1e-15 * max(1.0, abs(want)):
                    return False
    return True


PINS = [_pin_library, _pin_closed_forms, _pin_invariants, _pin_brute_force]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_softmax_rows_pins(pin):
    assert pin(softmax_rows)


def test_empty_row_count():
    assert softmax_rows(np.zeros((0, 17))).shape == (0, 17)
    assert split_softmax_model(np.zeros((0, 17)), 4).shape == (0, 17)


def _mutant_no_max(x):
    e = np.exp(np.asarray(x, dtype=np.float64))
    return e / e.sum(axis=1, keepdims=True)


def _mutant_column_sum(x):
    x = np.asarray(x, dtype=np.float64)
    e = np.exp(x - x.max(axis=1, keepdims=True))
    return e / e.sum(axis=0, keepdims=True)


def _mutant_global_max(x):
    x = np.asarray(x, dtype=np.float64)
    e = np.exp(x - x.max())
    return e / e.sum(axis=1, keepdims=True)


def _mutant_sign(x):
    x = np.asarray(x, dtype=np.float64)
    e = np.exp(-(x - x.max(axis=1, keepdims=True)))
    return e / e.sum(axis=1, keepdims=True)


def _mutant_float32(x):
    x = np.asarray(x, dtype=np.float32)
    e = np.exp(x - x.max(axis=1, keepdims=True))
    return (e / e.sum(axis=1, keepdims=True)).astype(np.float64)


@pytest.mark.parametrize("mutant", [_mutant_no_max, _mutant_column_sum, _mutant_global_max,
                                    _mutant_sign, _mutant_float32],
                         ids=lambda m: m.__name__)
def test_pins_reject_mutants(mutant):
    with np.errstate(all="ignore"):
        assert not all(pin(mutant) for pin in PINS)


# --------------------------------------------------------------------------
# The split (A2) model: partial statistics, rescaled merge, re-read.

@pytest.mark.parametrize("n,chunk", [(1, 256), (255, 256), (256, 256), (257, 256), (1000, 64),
                                     (4097, 1024), (300, 1), (50, 4096)])
def test_split_model_equals_row_softmax(n, chunk):
    rng = np.random.default_rng(n + chunk)
    x = rng.standard_normal((3, n)) * 5.0
    x[1] += np.linspace(0.0, 40.0, n)  # later chunks hold the row maximum
    y = split_softmax_model(x, chunk)
    assert np.allclose(y, softmax_rows(x), rtol=1e-13, atol=0)
    assert np.allclose(y.sum(axis=1), 1.0, rtol=0, atol=1e-13)


def test_split_model_catches_local_normalisation():
    rng = np.random.default_rng(7)
    x = rng.standard_normal((2, 700))
    good = softmax_rows(x)
    bad = split_softmax_model(x, 256, bugs=("local_normalise",))
    assert not np.allclose(bad, good, rtol=1e-6, atol=0)
    assert np.allclose(bad.sum(axis=1), 3.0)  # three chunks, each summing to one
    # With a single chunk the mistake is invisible, as the page's method implies.
    assert np.allclose(split_softmax_model(x, 1024, bugs=("local_normalise",)), good,
                       rtol=1e-13, atol=0)


def test_split_model_rejects_unknown_bug():
    with pytest.raises(ValueError):
        split_softmax_model(np.zeros((1, 4)), 2, bugs=("nope",))


# --------------------------------------------------------------------------
# Masked entries (-inf): the mass of a row is that of its unmasked entries.

def test_masked_entries_reduce_to_softmax_of_the_rest():
    # Softmax over a row with -inf entries equals the library softmax of the
    # finite entries, with exact zeros in the masked places; a row with every
    # entry masked has no mass and returns zeros (never NaN).
    rng = np.random.default_rng(11)
    x = rng.standard_normal((4, 40)) * 3.0
    keep = rng.random((4, 40)) < 0.6
    keep[:, 7] = True          # at least one finite entry per row
    x[~keep] = -np.inf
    x[3, :] = -np.inf          # a fully masked row
    y = softmax_rows(x)
    assert np.all(np.isfinite(y))
    assert np.array_equal(y[~keep], np.zeros(int((~keep).sum())))
    for r in range(3):
        assert np.allclose(y[r, keep[r]], scipy.special.softmax(x[r, keep[r]]), rtol=1e-13, atol=0)
    assert np.array_equal(y[3], np.zeros(40))


@pytest.mark.parametrize("chunk", [1, 4, 8, 16])
def test_split_model_with_masked_chunks(chunk):
    # Whole chunks of -inf (the empty state in the merge), masked runs that
    # straddle chunk edges, and a fully masked row.
    rng = np.random.default_rng(chunk)
    x = rng.standard_normal((3, 64)) * 2.0
    x[0, :16] = -np.inf
    x[1, 5:37] = -np.inf
    x[2, :] = -np.inf
    y = split_softmax_model(x, chunk)
    assert np.all(np.isfinite(y))
    assert np.allclose(y, softmax_rows(x), rtol=1e-13, atol=0)
    assert np.array_equal(y[2], np.zeros(64))
