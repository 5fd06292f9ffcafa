"""Plain FP64 reference for attention over packed variable-length sequences.

TEST INFRASTRUCTURE ONLY (see the package docstring): the product path never
imports this module.

The workshops page lists padding lengths among the attention contract's
explicit non-features ("Scope and contracts", paragraph after the table);
this is the usual packed form of them.  B sequences are concatenated along
the token axis: q is [total_q, H, D] and k, v are [total_k, Hkv, D]; sequence
b owns query rows cu_q[b] .. cu_q[b+1]-1 and key rows cu_k[b] .. cu_k[b+1]-1.
Each sequence is attended on its own, exactly as oracle.attention_rows
defines it (causal keys aligned to the end of the sequence's query block),
with K/V head h // (H // Hkv) for query head h.  The row states are returned
head-major, [H, total_q].
"""

import numpy as np

from .attention import NEG_INF, attention_rows


def attention_varlen(q, k, v, cu_q, cu_k, causal, scale):
    """Returns (out [total_q, H, D], m [H, total_q], l [H, total_q])."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    total_q, h_, d = q.shape
    hkv = k.shape[1]
    group = h_ // hkv
    out = np.zeros((total_q, h_, v.shape[2]))
    m = np.full((h_, total_q), NEG_INF)
    l = np.zeros((h_, total_q))
    for b in range(len(cu_q) - 1):
        q0, q1 = int(cu_q[b]), int(cu_q[b + 1])
        k0, k1 = int(cu_k[b]), int(cu_k[b + 1])
        for h in range(h_):
            o, mm, ll = attention_rows(q[q0:q1, h], k[k0:k1, h // group], v[k0:k1, h // group],
                                       causal, scale)
            out[q0:q1, h] = o
            m[h, q0:q1] = mm
            l[h, q0:q1] = ll
    return out, m, l
