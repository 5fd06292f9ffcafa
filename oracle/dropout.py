"""Plain FP64 reference for attention with dropout on the probabilities.

TEST INFRASTRUCTURE ONLY (see the package docstring): the product path never
imports this module.

The workshops page lists dropout among the attention contract's explicit
non-features ("Scope and contracts", paragraph after the table).  What is
computed here, per head bh = b * H + h, query row i and key j:

    w_ij  = exp(s_ij - m_i) on visible keys (s, m, l as oracle.attention_rows)
    l_i   = sum_j w_ij                       (dropout does not change l)
    out_i = sum_j w_ij * keep_ij * V_j / l_i * 65536 / (65536 - T)

where keep_ij comes from the counter-based generator Philox4x64-10 (Salmon,
Moraes, Dror and Shaw, "Parallel random numbers: as easy as 1, 2, 3",
SC 2011).  The generator runs on the 4-word counter (j // 16, i, bh,
offset) with the 2-word key (seed, 0); its four 64-bit outputs hold sixteen
16-bit fields, field t at bits 16 * (t % 4) of output t // 4, and key j is
kept iff field j % 16 >= T, T = round(p * 65536).  The drop probability is
therefore T / 65536, and the factor 65536 / (65536 - T) makes every output
unbiased.  philox4x64 is written from the paper's definition (ten rounds;
each round multiplies counter words 0 and 2 by the two multipliers, keeps
both 128-bit products' halves and mixes them with words 1, 3 and the key;
the key is bumped by the two Weyl constants between rounds).
"""

import numpy as np

from .attention import attention_rows

_M0 = 0xD2E7470EE14C6C93
_M1 = 0xCA5A826395121157
_W0 = 0x9E3779B97F4A7C15
_W1 = 0xBB67AE8584CAA73B
_MASK32 = np.uint64(0xFFFFFFFF)


def _mulhilo64(a, b):
    """(hi, lo) of the 128-bit product of the constant a and uint64 array b."""
    b = np.asarray(b, dtype=np.uint64)
    a_lo, a_hi = np.uint64(a & 0xFFFFFFFF), np.uint64(a >> 32)
    b_lo, b_hi = b & _MASK32, b >> np.uint64(32)
    ll = a_lo * b_lo
    lh = a_lo * b_hi
    hl = a_hi * b_lo
    hh = a_hi * b_hi
    mid = (ll >> np.uint64(32)) + (lh & _MASK32) + (hl & _MASK32)
    lo = (ll & _MASK32) | ((mid & _MASK32) << np.uint64(32))
    hi = hh + (lh >> np.uint64(32)) + (hl >> np.uint64(32)) + (mid >> np.uint64(32))
    return hi, lo


def philox4x64(c0, c1, c2, c3, k0, k1, rounds=10):
    """Philox4x64 on uint64 arrays (broadcast); returns its four output words."""
    with np.errstate(over="ignore"):
        c = [np.asarray(x, dtype=np.uint64) for x in (c0, c1, c2, c3)]
        k0 = np.uint64(k0)
        k1 = np.uint64(k1)
        for r in range(rounds):
            if r:
                k0 = k0 + np.uint64(_W0)
                k1 = k1 + np.uint64(_W1)
            hi0, lo0 = _mulhilo64(_M0, c[0])
            hi1, lo1 = _mulhilo64(_M1, c[2])
            c = [hi1 ^ c[1] ^ k0, lo1, hi0 ^ c[3] ^ k1, lo0]
    return c


def threshold(p):
    """The 16-bit drop threshold T = round(p * 65536) for 0 <= p < 1."""
    t = int(np.floor(p * 65536.0 + 0.5))
    if not 0 <= t <= 65535:
        raise ValueError("p must satisfy 0 <= round(p * 65536) <= 65535")
    return t


def keep_mask(bh, nq, nk, p, seed, offset):
    """Bool [nq, nk]: which keys row i of head bh keeps."""
    t = threshold(p)
    i = np.arange(nq, dtype=np.uint64)[:, None]
    j = np.arange(nk, dtype=np.uint64)[None, :]
    words = philox4x64(j // np.uint64(16), i, np.uint64(bh), np.uint64(offset), seed, 0)
    field_idx = (j % np.uint64(16)).astype(np.int64)
    out = np.zeros((nq, nk), dtype=np.uint64)
    for w in range(4):
        sel = (field_idx // 4) == w
        shift = (np.uint64(16) * (j % np.uint64(4))).astype(np.uint64)
        vals = (words[w] >> shift) & np.uint64(0xFFFF)
        out = np.where(sel, vals, out)
    return out >= np.uint64(t)


def attention_dropout(q, k, v, causal, scale, p, seed, offset=0):
    """Batched [B, H, N, D]; returns (out, m, l) with the row states of the
    plain softmax (dropout does not change m, l)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    b_, h_, nq, _ = q.shape
    nk = k.shape[2]
    t = threshold(p)
    gain = 65536.0 / (65536.0 - t)
    out = np.zeros((b_, h_, nq, v.shape[3]))
    m = np.full((b_, h_, nq), -np.inf)
    l = np.zeros((b_, h_, nq))
    for b in range(b_):
        for h in range(h_):
            keep = keep_mask(b * h_ + h, nq, nk, p, seed, offset)
            # Weights exp(s - m) of the visible keys, via the plain softmax
            # on one-hot values: attention_rows with V = I gives w / l.
            probs, mm, ll = attention_rows(q[b, h], k[b, h], np.eye(nk), causal, scale)
            out[b, h] = (probs * keep) @ v[b, h] * gain
            m[b, h], l[b, h] = mm, ll
    return out, m, l
