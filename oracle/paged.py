"""Plain FP64 reference for attention over a paged key/value cache.

TEST INFRASTRUCTURE ONLY (see the package docstring): the product path never
imports this module.

A paged cache stores each sequence's keys and values in fixed-size pages that
need not be contiguous or in order: ``k_cache`` and ``v_cache`` are
[num_pages, Hkv, page_size, D]; ``block_table[b, p]`` names the physical page
that holds keys p * page_size .. (p + 1) * page_size - 1 of sequence b, and
``seq_lens[b]`` is how many keys sequence b has.  The pages name a KV-cache
slice only as planned work (workshops page, the plan for week +3); this
layout is the usual one.  Attention itself is the plain definition of
oracle.attention_rows on the gathered keys, with K/V head h // (H // Hkv)
for query head h, causal alignment to the end of each sequence and an
optional sliding window.
"""

import numpy as np

from .attention import attention_rows


def gather_pages(cache, table_row, head, n, page_size):
    """The first n rows of one head of a sequence, in key order: [n, D]."""
    cache = np.asarray(cache)
    rows = []
    for j in range(n):
        page = int(table_row[j // page_size])
        rows.append(cache[page, head, j % page_size])
    if not rows:
        return np.zeros((0, cache.shape[3]), dtype=np.float64)
    return np.asarray(rows, dtype=np.float64)


def attention_paged(q, k_cache, v_cache, block_table, seq_lens, causal, scale, window=0):
    """q: [B, H, Nq, D]; returns (out [B, H, Nq, D], m [B, H, Nq], l [B, H, Nq])."""
    q = np.asarray(q, dtype=np.float64)
    b_, h_, nq, d = q.shape
    hkv = k_cache.shape[1]
    page_size = k_cache.shape[2]
    group = h_ // hkv
    out = np.zeros((b_, h_, nq, d))
    m = np.full((b_, h_, nq), -np.inf)
    l = np.zeros((b_, h_, nq))
    for b in range(b_):
        n = int(seq_lens[b])
        for hk in range(hkv):
            k = gather_pages(k_cache, block_table[b], hk, n, page_size)
            v = gather_pages(v_cache, block_table[b], hk, n, page_size)
            for h in range(hk * group, hk * group + group):
                out[b, h], m[b, h], l[b, h] = attention_rows(q[b, h], k, v, causal, scale,
                                                             window=window)
    return out, m, l
