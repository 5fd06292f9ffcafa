"""Plain FP64 reference for row softmax and the wide-row split softmax.

TEST INFRASTRUCTURE ONLY (see the package docstring): the product path never
imports this module.

What is computed, for each row x of a contiguous [M, N] matrix:

    softmax(x)_j = exp(x_j - max x) / sum_k exp(x_k - max x)

the plain two-pass definition (max, then exponentials and their sum).  The
workshops page ("Intermediate and advanced kernel workshops", section
"Scope and contracts") states the split_softmax contract: contiguous 2D
input, the same shape and dtype out, 1 to 131072 columns, an empty row count
allowed, chunk sizes 256 / 1024 / 4096.  The answer-key page ("Compare
reasoning after your own attempt") gives its method in row A2 of its table:
partial statistics per chunk, a rescaled merge, then a re-read that
normalises, all on one stream; the same row names the mistake to avoid
(chunk-local probabilities concatenated as if they were normalised over the
whole row).  Its worked answer A2 sizes the per-call scratch:
M = 4, N = 32769, C = 1024 needs T = 33 chunks and 8*4*(33+1) = 1088 bytes,
i.e. two FP32 numbers (m, l) per chunk plus two per row.

``split_softmax_model`` follows those three steps in FP64, chunk by chunk,
with a switch that plants the page's mistake so tests can show it is caught.
"""

import math

import numpy as np

NEG_INF = float("-inf")


def softmax_rows(x):
    """Two-pass FP64 softmax of every row of a 2D array (M may be 0)."""
    x = np.asarray(x, dtype=np.float64)
    if x.ndim != 2:
        raise ValueError("softmax_rows expects a 2D array")
    if x.shape[0] == 0:
        return np.zeros_like(x)
    m = x.max(axis=1, keepdims=True)          # pass 1: row maximum
    # Masked entries are -inf: they weigh exp(-inf) = 0.  A row with every
    # entry masked has no mass at all; its reference is pinned at 0 and it
    # returns zeros instead of NaN ("Kernel Notes & Checklist", gotchas
    # ledger: empty rows are pinned so they cannot produce NaN).
    ref = np.where(np.isneginf(m), 0.0, m)
    e = np.exp(x - ref)                       # pass 2: exponentials ...
    s = e.sum(axis=1, keepdims=True)          # ... and their sum
    return np.divide(e, s, out=np.zeros_like(e), where=s > 0)


def num_chunks(n, chunk):
    """T = ceil(N / C): chunks per row (answer-key page, worked answer A2)."""
    if chunk <= 0:
        raise ValueError("chunk must be positive")
    return -(-int(n) // int(chunk))


def scratch_bytes(m, n, chunk):
    """Per-call scratch of the split softmax: FP32 (m, l) per chunk and per row.

    8 * M * (T + 1) bytes; the answer-key page's worked answer A2 prints 1088
    for M = 4, N = 32769, C = 1024.
    """
    return 8 * int(m) * (num_chunks(n, chunk) + 1)


def split_softmax_model(x, chunk, bugs=()):
    """The A2 method of the answer-key page, in FP64.

    Step 1, per chunk c of each row: partial maximum m_c and partial sum
        l_c = sum_{j in c} exp(x_j - m_c).
    Step 2, per row: merge the T partial states by re-expressing each
        relative to the common maximum (answer-key row A1):
        m = max_c m_c,  l = sum_c l_c * exp(m_c - m).
    Step 3, per chunk again: y_j = exp(x_j - m) / l.

    ``bugs`` plants the page's mistake, for tests only:
      "local_normalise" -- each chunk normalised by its own (m_c, l_c) and the
                           pieces concatenated, skipping the merge.
    """
    bugs = set(bugs)
    unknown = bugs - {"local_normalise"}
    if unknown:
        raise ValueError(f"unknown planted bug(s): {sorted(unknown)}")
    x = np.asarray(x, dtype=np.float64)
    mrows, n = x.shape
    t = num_chunks(n, chunk) if n else 0
    y = np.zeros_like(x)
    for r in range(mrows):
        parts = []
        for c in range(t):
            seg = x[r, c * chunk:(c + 1) * chunk]
            mc = seg.max()
            ref = 0.0 if mc == NEG_INF else mc  # an all -inf chunk is the empty state
            parts.append((mc, math.fsum(math.exp(v - ref) for v in seg)))
        if "local_normalise" in bugs:
            for c, (mc, lc) in enumerate(parts):
                seg = x[r, c * chunk:(c + 1) * chunk]
                y[r, c * chunk:(c + 1) * chunk] = np.exp(seg - mc) / lc
            continue
        m = max(mc for mc, _ in parts)
        ref = 0.0 if m == NEG_INF else m
        l = math.fsum(lc * math.exp(mc - ref) for mc, lc in parts)
        y[r] = np.exp(x[r] - ref) / l if l > 0 else 0.0
    return y
