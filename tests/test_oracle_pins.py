"""Pins for the FP64 oracle, checked against what the pages and mathematics fix.

Every check here is independent of the oracle's own arithmetic: values the
pages print (tests/golden/worked_examples.json), closed forms (prefix means,
Nk = 1), invariants (shift, permutation, convexity, merge split-invariance)
and 50-digit brute force on tiny inputs.  ``test_pins_reject_mutants`` runs
the same pins against copies of the oracle with one plausible mistake planted
each, to show that every such mistake fails at least one pin.
"""

import itertools
import json
import math
import os

import mpmath
import numpy as np
import pytest

import oracle
from oracle import (EMPTY_STATE, attention, attention_rows, merge_state_of,
                    online_merge, streaming_model, visible_mask)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_examples.json")


def _golden():
    with open(GOLDEN) as f:
        return json.load(f)


def _num(x):
    if isinstance(x, str):
        return float(eval(x, {"__builtins__": {}},
                          {"log": math.log, "exp": math.exp, "inf": math.inf}))
    return float(x)


# --------------------------------------------------------------------------
# Worked examples printed on the answer-key page.
# --------------------------------------------------------------------------

def _a3_inputs():
    g = _golden()["a3_six_or_seven"]
    logits = np.array([_num(x) for x in g["logits"]])
    values = np.array(g["values"])
    # D = 1, Q = [1], K = logits, scale = 1 gives exactly these logits.
    q = np.ones((1, 1))
    k = logits[:, None]
    v = values[:, None]
    return q, k, v, g


def test_a3_worked_example_two_pass():
    q, k, v, g = _a3_inputs()
    out, m, l = attention_rows(q, k, v, causal=False, scale=1.0)
    assert abs(out[0, 0] - g["expected"]) <= 1e-14
    assert m[0] == math.log(2)
    assert abs(l[0] - 2.0) <= 1e-15  # exp(-ln2) * 2 + 1


@pytest.mark.parametrize("block_n", [1, 2, 3, 4])
def test_a3_streaming_model_gives_six(block_n):
    q, k, v, g = _a3_inputs()
    out = streaming_model(q, k, v, False, 1.0, block_n)
    assert abs(out[0, 0] - g["expected"]) <= 1e-14


@pytest.mark.parametrize("block_n,expected_key", [
    (1, "expected_if_a_not_rescaled"),
    (2, "expected_if_a_not_rescaled"),
    (3, "expected"),  # one tile: the missing rescale never fires
])
def test_a3_missing_alpha_on_a_gives_seven(block_n, expected_key):
    q, k, v, g = _a3_inputs()
    out = streaming_model(q, k, v, False, 1.0, block_n, bugs={"no_alpha_on_a"})
    assert abs(out[0, 0] - g[expected_key]) <= 1e-14


def test_a1_merge_worked_example():
    g = _golden()["a1_merge"]
    m, l = online_merge(*g["state_1"], *g["state_2"])
    assert m == g["expected_m"]
    assert abs(l - _num(g["expected_l"])) <= 2 ** -52 * 2
    # Commutative.
    m2, l2 = online_merge(*g["state_2"], *g["state_1"])
    assert (m2, l2) == (m, l)


def test_a1_empty_with_empty_is_empty_not_nan():
    g = _golden()["a1_empty_with_empty"]
    m, l = online_merge(*[_num(x) for x in g["state_1"]],
                        *[_num(x) for x in g["state_2"]])
    assert m == _num(g["expected_m"]) and l == g["expected_l"]
    assert (m, l) == EMPTY_STATE
    assert not math.isnan(m) and not math.isnan(l)


# --------------------------------------------------------------------------
# Merge invariants (A1): identity, split invariance, associativity.
# --------------------------------------------------------------------------

def test_merge_identity_is_exact():
    rng = np.random.default_rng(1)
    for _ in range(100):
        m, l = float(rng.normal() * 30), float(rng.uniform(0.1, 50))
        assert online_merge(m, l, *EMPTY_STATE) == (m, l)
        assert online_merge(*EMPTY_STATE, m, l) == (m, l)


def test_merge_split_invariance_and_associativity():
    rng = np.random.default_rng(2)
    for n in [1, 2, 5, 17]:
        x = rng.normal(size=n) * 20
        whole = merge_state_of(x)
        for cut in range(n + 1):
            st = online_merge(*merge_state_of(x[:cut]), *merge_state_of(x[cut:]))
            assert st[0] == whole[0]
            assert abs(st[1] - whole[1]) <= 1e-13 * whole[1]
    for _ in range(50):
        a, b, c = (merge_state_of(rng.normal(size=4) * 10) for _ in range(3))
        left = online_merge(*online_merge(*a, *b), *c)
        right = online_merge(*a, *online_merge(*b, *c))
        assert left[0] == right[0]
        assert abs(left[1] - right[1]) <= 1e-14 * left[1]


def test_merge_state_matches_fsum_of_exponentials():
    # sum exp(x) = l * e^m, checked against a 50-digit sum.
    rng = np.random.default_rng(3)
    mpmath.mp.dps = 50
    for n in [1, 3, 8]:
        x = rng.normal(size=n) * 5
        m, l = merge_state_of(x)
        exact = mpmath.fsum(mpmath.exp(mpmath.mpf(t)) for t in x)
        assert abs(mpmath.mpf(l) * mpmath.exp(m) - exact) <= 1e-14 * exact


def test_merge_arrays_elementwise():
    m1 = np.array([2.0, -np.inf, 0.0, -np.inf])
    l1 = np.array([2.0, 0.0, 3.0, 0.0])
    m2 = np.array([4.0, 1.0, -np.inf, -np.inf])
    l2 = np.array([1.0, 5.0, 0.0, 0.0])
    m, l = online_merge(m1, l1, m2, l2)
    assert list(m) == [4.0, 1.0, 0.0, -np.inf]
    assert abs(l[0] - (1 + 2 * math.exp(-2))) <= 4e-16
    assert list(l[1:]) == [5.0, 3.0, 0.0]


# --------------------------------------------------------------------------
# The pin suite for an attention implementation with the oracle's signature.
# Each pin returns None when it holds and a message when it fails.
# --------------------------------------------------------------------------

def _brute_force(q, k, v, causal, scale):
    """softmax(scale Q K^T) V by definition, 50 digits, no max subtraction.

    Visibility is enumerated with explicit loops from the causal rule of the
    workshops page ("diagonal included"), keys aligned to the end of the
    query block when Nq != Nk.
    """
    mpmath.mp.dps = 50
    nq, d = q.shape
    nk, dv = v.shape
    out = np.zeros((nq, dv))
    for i in range(nq):
        den = mpmath.mpf(0)
        num = [mpmath.mpf(0)] * dv
        for j in range(nk):
            if causal and j - (nk - nq) > i:
                continue
            s = mpmath.mpf(scale) * mpmath.fsum(
                mpmath.mpf(float(q[i, t])) * mpmath.mpf(float(k[j, t]))
                for t in range(d))
            w = mpmath.exp(s)
            den += w
            num = [num[t] + w * mpmath.mpf(float(v[j, t])) for t in range(dv)]
        if den != 0:
            out[i] = [float(num[t] / den) for t in range(dv)]
    return out


def pin_brute_force(fn):
    rng = np.random.default_rng(4)
    shapes = [(1, 1, 1, 1), (3, 3, 2, 2), (4, 6, 3, 2), (6, 4, 2, 3), (5, 5, 4, 1),
              (2, 7, 1, 2)]
    for (nq, nk, d, dv), causal in itertools.product(shapes, [False, True]):
        q = rng.normal(size=(nq, d))
        k = rng.normal(size=(nk, d))
        v = rng.normal(size=(nk, dv))
        scale = 0.7
        got = fn(q, k, v, causal, scale)[0]
        want = _brute_force(q, k, v, causal, scale)
        err = np.max(np.abs(got - want)) if got.size else 0.0
        if not err <= 1e-13:
            return f"brute force {nq}x{nk}x{d} causal={causal}: err {err}"
    return None


def pin_prefix_means(fn):
    # Q = 0 gives equal weights; with V[j] = (j, j^2) row i of causal
    # attention is the mean over its visible prefix, a closed form.
    for nq, nk in [(9, 9), (5, 9), (9, 5), (1, 1), (16, 16)]:
        d = 3
        q = np.zeros((nq, d))
        k = np.random.default_rng(5).normal(size=(nk, d))
        j = np.arange(nk, dtype=np.float64)
        v = np.stack([j, j * j], axis=1)
        for causal in [False, True]:
            out = fn(q, k, v, causal, 0.125)[0]
            for i in range(nq):
                n = nk if not causal else min(nk, max(0, i + (nk - nq) + 1))
                want = [0.0, 0.0] if n == 0 else [(n - 1) / 2, (n - 1) * (2 * n - 1) / 6]
                if not np.allclose(out[i], want, rtol=0, atol=1e-12):
                    return f"prefix mean {nq}x{nk} causal={causal} row {i}: {out[i]} vs {want}"
    return None


def pin_single_key(fn):
    # Nk = 1: the only visible key gets weight 1 whatever its score.
    rng = np.random.default_rng(6)
    q = rng.normal(size=(4, 3)) * 10
    k = rng.normal(size=(1, 3)) * 10
    v = rng.normal(size=(1, 5))
    out = fn(q, k, v, False, 1.0)[0]
    if not np.array_equal(out, np.repeat(v, 4, axis=0)):
        return "Nk = 1 is not the value row"
    return None


def pin_shift_invariance(fn):
    # Adding c to every logit of a row (through an extra feature column)
    # leaves softmax unchanged; c = 1000 overflows exp() unless the max is
    # subtracted.
    rng = np.random.default_rng(7)
    q = rng.normal(size=(6, 3))
    k = rng.normal(size=(8, 3))
    v = rng.normal(size=(8, 2))
    base = fn(q, k, v, False, 1.0)[0]
    for c in [1.0, 50.0, 1000.0]:
        q2 = np.concatenate([q, np.ones((6, 1))], axis=1)
        k2 = np.concatenate([k, np.full((8, 1), c)], axis=1)
        got = fn(q2, k2, v, False, 1.0)[0]
        if not np.all(np.isfinite(got)) or np.max(np.abs(got - base)) > 1e-10:
            return f"shift by {c} changed the output"
    return None


def pin_permutation_and_convexity(fn):
    rng = np.random.default_rng(8)
    q = rng.normal(size=(5, 4))
    k = rng.normal(size=(7, 4))
    v = rng.normal(size=(7, 3))
    out = fn(q, k, v, False, 0.5)[0]
    perm = rng.permutation(7)
    out2 = fn(q, k[perm], v[perm], False, 0.5)[0]
    if np.max(np.abs(out - out2)) > 1e-13:
        return "noncausal output depends on key order"
    if np.any(out < v.min(axis=0) - 1e-15) or np.any(out > v.max(axis=0) + 1e-15):
        return "output outside the convex hull of V"
    return None


def pin_worked_example(fn):
    q, k, v, g = _a3_inputs()
    out = fn(q, k, v, False, 1.0)[0]
    if abs(out[0, 0] - g["expected"]) > 1e-14:
        return f"A3 worked example gives {out[0, 0]}"
    return None


def pin_merge_state(fn):
    # The returned (m, l) is the A1 state of the row's scaled logits.
    rng = np.random.default_rng(9)
    q = rng.normal(size=(3, 2))
    k = rng.normal(size=(5, 2))
    v = rng.normal(size=(5, 1))
    _, m, l = fn(q, k, v, False, 0.8)
    for i in range(3):
        st = merge_state_of([0.8 * float(q[i] @ k[j]) for j in range(5)])
        if abs(m[i] - st[0]) > 1e-14 or abs(l[i] - st[1]) > 1e-13:
            return f"row {i} state {(m[i], l[i])} vs {st}"
    return None


PINS = [pin_worked_example, pin_brute_force, pin_prefix_means, pin_single_key,
        pin_shift_invariance, pin_permutation_and_convexity, pin_merge_state]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_oracle_passes_pin(pin):
    assert pin(attention_rows) is None


# Plausible mistakes, planted in copies of the oracle on the CPU.
def _mutant(kind):
    def fn(q, k, v, causal, scale):
        q, k, v = (np.asarray(t, dtype=np.float64) for t in (q, k, v))
        nq, nk = q.shape[0], k.shape[0]
        sc = 1.0 if kind == "drop_scale" else scale
        s = sc * (q @ k.T)
        if kind == "transpose_k" and s.shape[0] == s.shape[1]:
            s = s.T
        rows = np.arange(nq)[:, None]
        cols = np.arange(nk)[None, :]
        if causal:
            if kind == "causal_direction":
                vis = cols >= rows + (nk - nq)
            elif kind == "causal_no_offset":
                vis = cols <= rows
            elif kind == "causal_strict":
                vis = cols < rows + (nk - nq)
            else:
                vis = cols <= rows + (nk - nq)
        else:
            vis = np.ones((nq, nk), dtype=bool)
        fill = 0.0 if kind == "pad_zero" else -np.inf
        s = np.where(vis, s, fill)
        with np.errstate(all="ignore"):
            m = s.max(axis=1)
            if kind == "no_max":
                e = np.exp(s)
            else:
                e = np.exp(s - np.where(np.isfinite(m), m, 0)[:, None])
            l = e.sum(axis=1)
            a = e @ v
            if kind == "no_normalise":
                out = a
            else:
                out = np.where(l[:, None] > 0, a / np.where(l > 0, l, 1)[:, None], 0.0)
            if kind == "sign_flip":
                out = -out
        return out, m, l
    return fn


MUTANTS = ["drop_scale", "transpose_k", "causal_direction", "causal_no_offset",
           "causal_strict", "pad_zero", "no_max", "no_normalise", "sign_flip"]


@pytest.mark.parametrize("kind", MUTANTS)
def test_pins_reject_mutants(kind):
    fn = _mutant(kind)
    failures = [p.__name__ for p in PINS if p(fn) is not None]
    assert failures, f"mutant {kind} passed every pin"


def test_unmutated_copy_passes():
    fn = _mutant("none")
    assert all(p(fn) is None for p in PINS)


# --------------------------------------------------------------------------
# The streaming model against the two-pass definition, and the page's bugs.
# --------------------------------------------------------------------------

@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("nq,nk", [(13, 13), (7, 19), (19, 7), (1, 33)])
@pytest.mark.parametrize("block_n", [1, 4, 16, 64])
def test_streaming_model_equals_two_pass(causal, nq, nk, block_n):
    rng = np.random.default_rng(10)
    q = rng.normal(size=(nq, 8))
    k = rng.normal(size=(nk, 8)) + 0.3 * np.arange(nk)[:, None]
    v = rng.normal(size=(nk, 5))
    want = attention_rows(q, k, v, causal, 0.35)[0]
    got = streaming_model(q, k, v, causal, 0.35, block_n)
    assert np.max(np.abs(got - want)) <= 1e-12


def test_planted_pad_with_zero_is_caught():
    # Gotchas ledger: padded K columns scored 0 instead of -inf.
    rng = np.random.default_rng(11)
    q = rng.normal(size=(32, 16))
    k = rng.normal(size=(37, 16))
    v = rng.normal(size=(37, 16))
    want = attention_rows(q, k, v, False, 0.25)[0]
    bad = streaming_model(q, k, v, False, 0.25, 16, bugs={"pad_with_zero"})
    assert np.max(np.abs(bad - want)) > 1e-2


def test_planted_no_ghost_pin_gives_nan():
    # Causal with Nq > Nk leaves the first rows with no visible key.
    rng = np.random.default_rng(12)
    q = rng.normal(size=(8, 4))
    k = rng.normal(size=(3, 4))
    v = rng.normal(size=(3, 4))
    good = streaming_model(q, k, v, True, 0.5, 2)
    assert np.all(np.isfinite(good)) and np.all(good[:5] == 0)
    bad = streaming_model(q, k, v, True, 0.5, 2, bugs={"no_ghost_pin"})
    assert np.isnan(bad[:5]).all()


def test_planted_no_alpha_caught_on_rising_max():
    # Keys with a rising offset push the running max up on every tile.
    rng = np.random.default_rng(13)
    q = np.abs(rng.normal(size=(16, 8)))
    k = rng.normal(size=(64, 8)) + 0.1 * np.arange(64)[:, None]
    v = rng.normal(size=(64, 8))
    want = attention_rows(q, k, v, False, 0.3)[0]
    bad = streaming_model(q, k, v, False, 0.3, 16, bugs={"no_alpha_on_a"})
    assert np.max(np.abs(bad - want)) > 1e-1


# --------------------------------------------------------------------------
# Masks, batching and the empty cases.
# --------------------------------------------------------------------------

def test_visible_mask_counts_by_enumeration():
    for nq, nk in [(1, 1), (4, 4), (3, 7), (7, 3), (0, 5), (5, 0), (129, 130)]:
        for causal in [False, True]:
            mask = visible_mask(nq, nk, causal)
            assert mask.shape == (nq, nk)
            for i in range(nq):
                want = [causal is False or j + nq <= i + nk for j in range(nk)]
                assert list(mask[i]) == want


def test_batched_equals_per_head_and_empty_cases():
    rng = np.random.default_rng(14)
    q = rng.normal(size=(2, 3, 5, 4))
    k = rng.normal(size=(2, 3, 6, 4))
    v = rng.normal(size=(2, 3, 6, 4))
    out, m, l = attention(q, k, v, True, 0.5)
    for b in range(2):
        for h in range(3):
            o, mm, ll = attention_rows(q[b, h], k[b, h], v[b, h], True, 0.5)
            assert np.array_equal(out[b, h], o)
            assert np.array_equal(m[b, h], mm) and np.array_equal(l[b, h], ll)
    # Nk = 0: every row is empty.
    o, mm, ll = attention_rows(q[0, 0], k[0, 0][:0], v[0, 0][:0], False, 0.5)
    assert np.all(o == 0) and np.all(mm == -np.inf) and np.all(ll == 0)
    # B = 0.
    o, _, _ = attention(q[:0], k[:0], v[:0], False, 0.5)
    assert o.shape == (0, 3, 5, 4)


def test_rows_subset_matches_full():
    rng = np.random.default_rng(15)
    q = rng.normal(size=(50, 8))
    k = rng.normal(size=(50, 8))
    v = rng.normal(size=(50, 8))
    full = attention_rows(q, k, v, True, 0.3)[0]
    rows = np.array([0, 7, 49, 31])
    sub = attention_rows(q, k, v, True, 0.3, rows)[0]
    assert np.array_equal(sub, full[rows])


def test_oracle_imports_nothing_from_the_product():
    import ast
    import sys
    for path in (sys.modules["oracle.attention"].__file__, oracle.__file__):
        tree = ast.parse(open(path).read())
        for node in ast.walk(tree):
            if isinstance(node, ast.Import):
                names = [a.name for a in node.names]
            elif isinstance(node, ast.ImportFrom):
                names = [node.module or ""]
            else:
                continue
            for name in names:
                assert name.split(".")[0] in {"math", "numpy"} or node.level > 0, name
