"""Pins for the FP64 attention-backward oracle.

Independent of the oracle's arithmetic: the softmax VJP worked example the
answer-key page prints (item I2, tests/golden/worked_examples.json) and its
stated property for a constant upstream gradient; central finite
differences of the forward oracle; torch.autograd on a plain float64 CPU
attention written with library ops; and identities (rowsum(P * dP) equals
rowsum(dO * O)).  Planted mistakes (the page's unweighted reduction, a
dropped scale, a transposed product, a wrong causal mask) must each fail.
"""

import json
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import (attention, attention_backward, attention_backward_head, probabilities,
                    softmax_vjp)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_examples.json")


def test_i2_worked_example():
    g = json.load(open(GOLDEN))["i2_softmax_vjp"]
    y = np.array(g["y"])
    gg = np.array(g["g"])
    assert float((y * gg).sum()) == g["expected_dot"]
    assert np.array_equal(softmax_vjp(y, gg), np.array(g["expected_dx"]))


def test_i2_constant_gradient_gives_zero():
    # The page: a constant upstream gradient gives ~0 because y sums to one.
    y = np.array([[0.1, 0.2, 0.7], [0.5, 0.25, 0.25]])
    assert np.max(np.abs(softmax_vjp(y, np.full_like(y, 3.0)))) <= 1e-15


def test_i2_unweighted_reduction_is_caught():
    g = json.load(open(GOLDEN))["i2_softmax_vjp"]
    bad = softmax_vjp(np.array(g["y"]), np.array(g["g"]), bugs=("unweighted_reduction",))
    assert not np.allclose(bad, g["expected_dx"])


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _loss(q, k, v, do, causal, scale):
    out, _, _ = attention(q, k, v, causal, scale)
    return float((out * do).sum())


@pytest.mark.parametrize("nq,nk,d,causal", [(3, 3, 2, False), (4, 4, 3, True), (3, 5, 2, True),
                                            (5, 3, 4, True), (2, 6, 3, False)])
def test_finite_differences(nq, nk, d, causal):
    q = _rand((1, 1, nq, d), 1)
    k = _rand((1, 1, nk, d), 2)
    v = _rand((1, 1, nk, d), 3)
    do = _rand((1, 1, nq, d), 4)
    scale = 0.7
    dq, dk, dv = attention_backward(q, k, v, do, causal, scale)
    h = 1e-6
    for x, g in ((q, dq), (k, dk), (v, dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            x0 = x[idx]
            x[idx] = x0 + h
            fp = _loss(q, k, v, do, causal, scale)
            x[idx] = x0 - h
            fm = _loss(q, k, v, do, causal, scale)
            x[idx] = x0
            num[idx] = (fp - fm) / (2 * h)
        assert np.allclose(g, num, rtol=1e-6, atol=1e-8)


def _torch_grads(q, k, v, do, causal, scale):
    tq, tk, tv = (torch.tensor(t, dtype=torch.float64, requires_grad=True) for t in (q, k, v))
    s = scale * torch.matmul(tq, tk.transpose(-1, -2))
    nq, nk = q.shape[-2], k.shape[-2]
    if causal:
        i = torch.arange(nq)[:, None]
        j = torch.arange(nk)[None, :]
        s = s.masked_fill(j > i + (nk - nq), float("-inf"))
    p = torch.softmax(s, dim=-1)
    p = torch.nan_to_num(p, nan=0.0)  # rows with no visible key
    out = torch.matmul(p, tv)
    out.backward(torch.tensor(do, dtype=torch.float64))
    return tq.grad.numpy(), tk.grad.numpy(), tv.grad.numpy()


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("nq,nk,d", [(33, 33, 16), (17, 40, 8), (40, 17, 8)])
def test_matches_torch_autograd(causal, nq, nk, d):
    q = _rand((2, 2, nq, d), 11)
    k = _rand((2, 2, nk, d), 12)
    v = _rand((2, 2, nk, d), 13)
    do = _rand((2, 2, nq, d), 14)
    scale = d ** -0.5
    got = attention_backward(q, k, v, do, causal, scale)
    want = _torch_grads(q, k, v, do, causal, scale)
    for g, w in zip(got, want):
        assert np.allclose(g, w, rtol=1e-10, atol=1e-12)


def test_delta_identity():
    # rowsum(P * dP) = rowsum(dO * O): the backward kernels use the right side.
    q, k, v, do = (_rand((1, 1, 20, 8), s)[0, 0] for s in (21, 22, 23, 24))
    out, _, _ = attention(q[None, None], k[None, None], v[None, None], True, 0.5)
    p = probabilities(q, k, True, 0.5)
    assert np.allclose((p * (do @ v.T)).sum(axis=1), (do * out[0, 0]).sum(axis=1), rtol=1e-12)


def test_rows_without_keys_get_zero_gradient():
    # Causal Nq > Nk: the first Nq - Nk rows see no key.
    q, k, v, do = _rand((6, 4), 31), _rand((2, 4), 32), _rand((2, 4), 33), _rand((6, 4), 34)
    dq, dk, dv = attention_backward_head(q, k, v, do, True, 0.5)
    assert np.all(dq[:4] == 0)
    assert np.all(np.isfinite(dk)) and np.all(np.isfinite(dv))


def _mutants():
    def no_scale_dq(q, k, v, do, causal, scale):
        p = probabilities(q, k, causal, scale)
        ds = softmax_vjp(p, do @ v.T)
        return ds @ k, scale * (ds.T @ q), p.T @ do

    def unweighted(q, k, v, do, causal, scale):
        p = probabilities(q, k, causal, scale)
        ds = softmax_vjp(p, do @ v.T, bugs=("unweighted_reduction",))
        return scale * (ds @ k), scale * (ds.T @ q), p.T @ do

    def dv_untransposed(q, k, v, do, causal, scale):
        p = probabilities(q, k, causal, scale)
        ds = softmax_vjp(p, do @ v.T)
        return scale * (ds @ k), scale * (ds.T @ q), p @ do

    def causal_ignored(q, k, v, do, causal, scale):
        return attention_backward_head(q, k, v, do, False, scale)

    return [no_scale_dq, unweighted, dv_untransposed, causal_ignored]


@pytest.mark.parametrize("mutant", _mutants(), ids=lambda f: f.__name__)
def test_pins_reject_mutants(mutant):
    q, k, v, do = _rand((7, 4), 41), _rand((7, 4), 42), _rand((7, 4), 43), _rand((7, 4), 44)
    want = _torch_grads(q, k, v, do, True, 0.6)
    got = mutant(q, k, v, do, True, 0.6)
    assert not all(np.allclose(g, w, rtol=1e-8, atol=1e-10) for g, w in zip(got, want))
