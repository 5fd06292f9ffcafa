"""Plain FP64 reference for streaming (online-softmax) attention.

TEST INFRASTRUCTURE ONLY (see the package docstring): the product path never
imports this module.

What is computed, per batch b, head h and query row i (notation of the
answer-key page, row A3: running max m, running sum l, unnormalised output a):

    visible(i)  = { j < Nk : not causal  or  j <= i + (Nk - Nq) }
    s_j         = scale * sum_d Q[i, d] * K[j, d]          (FP64, materialised)
    m           = max_{j in visible(i)} s_j                 (pass 1)
    l           = sum_{j in visible(i)} exp(s_j - m)        (pass 2)
    a_d         = sum_{j in visible(i)} exp(s_j - m) V[j, d]
    out[i, d]   = a_d / l,   and out[i, :] = 0 when visible(i) is empty.

Sources: workshops page ("Intermediate and advanced kernel workshops"),
section "Scope and contracts", streaming_attention row: single-head
self-attention Q/K/V[N, D], scale 1/sqrt(D) (here an explicit argument),
diagonal included when causal.  Answer-key page ("Compare reasoning after your
own attempt"), closing note of "Reference tradeoffs to challenge": the
attention oracle materialises FP64 scores.  Where the pages are silent this
module reads them as follows: heads are batched as [B, H, N, D]; with Nq != Nk
the causal rule aligns the last query with the last key (key j is visible to
query i iff j <= i + Nk - Nq); a row with no visible key returns zeros with
row state (m, l) = (-inf, 0); the scale is an explicit argument.

The two-pass form above is the plain definition of softmax(scale Q K^T) V with
the maximum subtracted for stability ("Kernel Notes & Checklist", section 4,
"The gotchas ledger": masked scores are -inf before a max and contribute 0 to
a sum).  ``streaming_model`` follows the streaming algorithm itself, tile by
tile in the order the answer-key page gives it, with switches that plant the
mistakes the pages name; it exists so tests can show those mistakes are caught.

Query rows are evaluated in independent chunks only to bound memory: every
row's arithmetic is exactly the definition above.
"""

import math

import numpy as np

NEG_INF = float("-inf")

#: The empty merge state (no logits seen): sum exp(x) = l * e^m = 0.
#: Answer-key page, A1 row: empty-with-empty must not produce NaN.
EMPTY_STATE = (NEG_INF, 0.0)

_ROW_CHUNK_ELEMS = 1 << 24  # fp64 score elements materialised per chunk


def visible_mask(nq, nk, causal, rows=None, window=0):
    """Boolean [len(rows), nk]: True where key j is visible to query row i.

    Workshops page, "Scope and contracts": causal attention includes the
    diagonal (j <= i for Nq == Nk).  For Nq != Nk the keys are aligned to the
    end of the query block (j <= i + Nk - Nq), which reduces to the pages'
    rule when the two lengths agree.

    ``window`` > 0 (causal only) keeps the ``window`` keys that end at the
    row's diagonal: j > i + (Nk - Nq) - window.  The pages name sliding
    windows only as planned work; this is the usual reading.
    """
    if rows is None:
        rows = np.arange(nq)
    rows = np.asarray(rows, dtype=np.int64)
    j = np.arange(nk, dtype=np.int64)[None, :]
    if window and not causal:
        raise ValueError("a sliding window needs causal attention")
    if not causal:
        return np.ones((rows.shape[0], nk), dtype=bool)
    diag = rows[:, None] + (nk - nq)
    vis = j <= diag
    if window:
        vis &= j > diag - window
    return vis


def attention_rows(q, k, v, causal, scale, rows=None, window=0, mask=None):
    """Two-pass FP64 attention for one head, on the query rows ``rows``.

    q: [Nq, D], k: [Nk, D], v: [Nk, Dv] arrays (upcast exactly to float64 by
    the caller).  ``scale`` is the same value the kernel receives.

    Returns (out [R, Dv], m [R], l [R]) where (m, l) is the row's merge state
    in natural-log units: sum_j exp(s_j) = l * exp(m); (m, l) = (-inf, 0) and
    out = 0 for a row with no visible key.  ``window`` as in visible_mask;
    ``mask`` (bool [Nq, Nk], optional) further hides every key where it is
    False: an arbitrary mask, which the workshops page lists among the
    attention contract's non-features ("Scope and contracts").
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    nq, nk = q.shape[0], k.shape[0]
    if rows is None:
        rows = np.arange(nq)
    rows = np.asarray(rows, dtype=np.int64)
    scale = float(scale)

    out = np.zeros((rows.shape[0], v.shape[1]), dtype=np.float64)
    m_all = np.full(rows.shape[0], NEG_INF)
    l_all = np.zeros(rows.shape[0], dtype=np.float64)
    if nk == 0 or rows.shape[0] == 0:
        return out, m_all, l_all

    step = max(1, _ROW_CHUNK_ELEMS // nk)
    for c0 in range(0, rows.shape[0], step):
        r = rows[c0:c0 + step]
        # Scores for these rows, materialised in FP64.
        s = scale * (q[r] @ k.T)
        vis = visible_mask(nq, nk, causal, r, window)
        if mask is not None:
            vis = vis & np.asarray(mask, dtype=bool)[r]
        s = np.where(vis, s, NEG_INF)
        nonempty = vis.any(axis=1)

        # Pass 1: the row maximum over visible keys.
        m = np.full(r.shape[0], NEG_INF)
        m[nonempty] = s[nonempty].max(axis=1)

        # Pass 2: exponentials relative to the maximum; masked keys give 0.
        e = np.zeros_like(s)
        e[nonempty] = np.exp(s[nonempty] - m[nonempty, None])
        l = e.sum(axis=1)
        a = e @ v

        o = np.zeros_like(a)
        o[nonempty] = a[nonempty] / l[nonempty, None]
        out[c0:c0 + step] = o
        m_all[c0:c0 + step] = m
        l_all[c0:c0 + step] = l
    return out, m_all, l_all


def attention(q, k, v, causal, scale, window=0, mask=None):
    """Batched two-pass FP64 attention on [B, H, N, D] arrays.

    ``mask``: optional bool array broadcastable to [B, H, Nq, Nk].
    Returns (out [B, H, Nq, Dv], m [B, H, Nq], l [B, H, Nq]).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    b, h, nq, _ = q.shape
    out = np.zeros((b, h, nq, v.shape[3]), dtype=np.float64)
    m = np.full((b, h, nq), NEG_INF)
    l = np.zeros((b, h, nq), dtype=np.float64)
    for bi in range(b):
        for hi in range(h):
            mk = None
            if mask is not None:
                mk = np.broadcast_to(np.asarray(mask, dtype=bool),
                                     (b, h, nq, k.shape[2]))[bi, hi]
            o, mm, ll = attention_rows(q[bi, hi], k[bi, hi], v[bi, hi],
                                       causal, scale, window=window, mask=mk)
            out[bi, hi], m[bi, hi], l[bi, hi] = o, mm, ll
    return out, m, l


def merge_state_of(x):
    """The A1 summary of a list of logits: (max x, sum exp(x - max x)).

    Answer-key page, A1 row: a state (m, l) stands for sum_j exp(x_j) =
    l * e^m.  An empty list gives EMPTY_STATE.
    """
    x = [float(t) for t in x]
    if not x:
        return EMPTY_STATE
    m = max(x)
    if m == NEG_INF:
        return EMPTY_STATE
    return m, math.fsum(math.exp(t - m) for t in x)


def online_merge(m1, l1, m2, l2):
    """Merge two A1 states by re-expressing both relative to the larger max.

    Answer-key page, A1 row and its worked answer: merging (2, 2) with (4, 1)
    gives (4, 1 + 2 exp(-2)); the older state shrinks instead of overflowing;
    two empty states merge to the empty state, not to NaN.

    Works elementwise on scalars or equally shaped arrays; scalars come back as
    Python floats.
    """
    scalar = all(np.ndim(t) == 0 for t in (m1, l1, m2, l2))
    m1, l1, m2, l2 = (np.asarray(t, dtype=np.float64) for t in (m1, l1, m2, l2))
    m = np.maximum(m1, m2)
    empty = m == NEG_INF
    # Re-express relative to the common maximum; for an empty pair the common
    # maximum is -inf and the subtraction would be -inf - -inf = NaN, so the
    # result is the empty state by definition.
    ref = np.where(empty, 0.0, m)
    l = l1 * np.exp(m1 - ref) + l2 * np.exp(m2 - ref)
    m = np.where(empty, NEG_INF, m)
    l = np.where(empty, 0.0, l)
    if scalar:
        return float(m), float(l)
    return m, l


def streaming_model(q, k, v, causal, scale, block_n, bugs=()):
    """The streaming algorithm of the answer-key page (row A3), in FP64.

    One head; keys are visited in tiles of ``block_n`` (the last tile padded
    to full width), carrying per query row the running max m, running sum l
    and unnormalised output a.  On each tile:

        masked or padded scores  -> -inf               (gotchas ledger)
        m_new = max(m, rowmax(s))
        m_ref = m_new, or 0 where m_new is -inf         (ghost-row pin)
        alpha = exp(m - m_ref)
        p     = exp(s - m_ref)
        l     = alpha * l + rowsum(p)
        a     = alpha * a + p @ V_tile                  (A3: rescale a too)

    and finally out = a / l (0 where l == 0).

    ``bugs`` plants the mistakes the pages describe, for tests only:
      "no_alpha_on_a" -- a is not rescaled (answer-key A3: 7 instead of 6);
      "pad_with_zero" -- masked/padded scores take 0 instead of -inf
                         (gotchas ledger: padded K columns scored 0);
      "no_ghost_pin"  -- m_ref = m_new even when it is -inf (gotchas ledger:
                         ghost rows give NaN).
    """
    bugs = set(bugs)
    unknown = bugs - {"no_alpha_on_a", "pad_with_zero", "no_ghost_pin"}
    if unknown:
        raise ValueError(f"unknown planted bug(s): {sorted(unknown)}")
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    nq, nk, dv = q.shape[0], k.shape[0], v.shape[1]
    if block_n < 1:
        raise ValueError("block_n must be >= 1")

    ntiles = -(-nk // block_n)
    pad = ntiles * block_n - nk
    kp = np.concatenate([k, np.zeros((pad, k.shape[1]))], axis=0)
    vp = np.concatenate([v, np.zeros((pad, dv))], axis=0)
    rows = np.arange(nq)
    fill = 0.0 if "pad_with_zero" in bugs else NEG_INF

    m = np.full(nq, NEG_INF)
    l = np.zeros(nq)
    a = np.zeros((nq, dv))
    with np.errstate(invalid="ignore"):
        for t in range(ntiles):
            j = t * block_n + np.arange(block_n)
            s = scale * (q @ kp[j].T)
            vis = (j < nk)[None, :]
            if causal:
                vis = vis & (j[None, :] <= rows[:, None] + (nk - nq))
            s = np.where(vis, s, fill)
            m_new = np.maximum(m, s.max(axis=1))
            if "no_ghost_pin" in bugs:
                m_ref = m_new
            else:
                m_ref = np.where(m_new == NEG_INF, 0.0, m_new)
            alpha = np.exp(m - m_ref)
            p = np.exp(s - m_ref[:, None])
            l = alpha * l + p.sum(axis=1)
            if "no_alpha_on_a" in bugs:
                a = a + p @ vp[j]
            else:
                a = alpha[:, None] * a + p @ vp[j]
            m = m_new
        out = np.zeros_like(a)
        ok = l != 0
        out[ok] = a[ok] / l[ok, None]
        # A NaN state must stay visible rather than be hidden by the l == 0 test.
        bad = np.isnan(l)
        out[bad] = np.nan
    return out
