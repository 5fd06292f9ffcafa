"""Plain FP64 reference for the attention backward pass.

TEST INFRASTRUCTURE ONLY (see the package docstring): the product path never
imports this module.

The forward pass per head is O = P V with P = softmax(scale * Q K^T) over the
visible keys of each row (the streaming_attention contract of the workshops
page, "Intermediate and advanced kernel workshops", section "Scope and
contracts"; oracle.attention computes it).  Given the upstream gradient dO,
the chain rule gives, per head:

    dV = P^T dO
    dP = dO V^T
    dS = softmax VJP of dP at P, row by row:  dS = P * (dP - rowsum(P * dP))
    dQ = scale * dS K
    dK = scale * dS^T Q

The row-wise softmax VJP is the workshops page's intermediate workshop I2
(softmax backward): one reduction of y*g, then y * (g - dot).  The answer-key
page ("Compare reasoning after your own attempt") works it for y = [.25, .75],
g = [2, -1]: dot = -.25, dx = [.5625, -.5625], and names the mistake of
reducing g alone (omitting the probability weighting); ``softmax_vjp`` can
plant that mistake for tests.  Masked keys have P = 0 and so receive no
gradient; rows with no visible key give zero gradients.
"""

import numpy as np

from .attention import visible_mask


def softmax_vjp(y, g, bugs=()):
    """Row-wise softmax vector-Jacobian product: y * (g - sum(y * g)).

    ``bugs`` may hold "unweighted_reduction" (the answer-key page's I2
    mistake: subtract sum(g) instead of sum(y * g)), for tests only.
    """
    bugs = set(bugs)
    unknown = bugs - {"unweighted_reduction"}
    if unknown:
        raise ValueError(f"unknown planted bug(s): {sorted(unknown)}")
    y = np.asarray(y, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    if "unweighted_reduction" in bugs:
        dot = g.sum(axis=-1, keepdims=True)
    else:
        dot = (y * g).sum(axis=-1, keepdims=True)
    return y * (g - dot)


def probabilities(q, k, causal, scale):
    """P for one head: masked, max-subtracted, row-normalised; empty rows 0."""
    s = scale * (q @ k.T)
    vis = visible_mask(q.shape[0], k.shape[0], causal)
    s = np.where(vis, s, -np.inf)
    p = np.zeros_like(s)
    rows = vis.any(axis=1)
    if rows.any():
        m = s[rows].max(axis=1, keepdims=True)
        e = np.exp(s[rows] - m)
        p[rows] = e / e.sum(axis=1, keepdims=True)
    return p


def attention_backward_head(q, k, v, do, causal, scale):
    """(dQ, dK, dV) for one head: q [Nq, D], k, v [Nk, D], do [Nq, D]."""
    q, k, v, do = (np.asarray(t, dtype=np.float64) for t in (q, k, v, do))
    p = probabilities(q, k, causal, float(scale))
    dv = p.T @ do
    dp = do @ v.T
    ds = softmax_vjp(p, dp)
    dq = float(scale) * (ds @ k)
    dk = float(scale) * (ds.T @ q)
    return dq, dk, dv


def attention_backward(q, k, v, do, causal, scale):
    """Batched (dQ, dK, dV) on [B, H, N, D] arrays."""
    q, k, v, do = (np.asarray(t, dtype=np.float64) for t in (q, k, v, do))
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for b in range(q.shape[0]):
        for h in range(q.shape[1]):
            dq[b, h], dk[b, h], dv[b, h] = attention_backward_head(
                q[b, h], k[b, h], v[b, h], do[b, h], causal, scale)
    return dq, dk, dv
