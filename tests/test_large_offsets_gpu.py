"""Element offsets past 2^31: heads whose rows start beyond the 32-bit range.

With B=260, H=64, N=1024, D=128 each of Q, K, V and O holds 2.18e9 > 2^31
elements, so the last heads start past the signed 32-bit range (and past
2^32 bytes).  The per-head bases are 64-bit; each kernel then addresses a
head with 32-bit offsets.  The first and the last heads are checked against
the oracle, in the launch configuration such a problem takes.
"""

import numpy as np
import pytest
import torch

import oracle
from online_softmax_streaming_amd import attn_bwd, attn_fwd, attn_fwd_stats, default_scale
from online_softmax_streaming_amd.workloads import random_dout, random_qkv

pytestmark = pytest.mark.gpu

B, H, N, D = 260, 64, 1024, 128
HEADS = [(0, 0), (B - 1, H - 2), (B - 1, H - 1)]
TOL = {"f32": 1e-5, "bf16": 1e-2}


def _np(t):
    return t.detach().to("cpu", torch.float64).numpy()


@pytest.fixture(scope="module")
def big_bf16():
    q, k, v = random_qkv(B, H, N, N, D, "bf16", seed=31, device="cuda")
    assert q.numel() > 2 ** 31
    yield q, k, v
    del q, k, v
    torch.cuda.empty_cache()


@pytest.mark.parametrize("causal", [False, True])
def test_forward_bf16_last_heads(big_bf16, causal):
    q, k, v = big_bf16
    scale = default_scale(D)
    out = attn_fwd(q, k, v, causal=causal, scale=scale)
    torch.cuda.synchronize()
    for b, h in HEADS:
        want, _, _ = oracle.attention_rows(_np(q[b, h]), _np(k[b, h]), _np(v[b, h]), causal, scale)
        err = float(np.max(np.abs(_np(out[b, h]) - want)))
        assert err <= TOL["bf16"], f"head ({b},{h}): max abs err {err}"
    del out


def test_backward_bf16_last_heads(big_bf16):
    q, k, v = big_bf16
    scale = default_scale(D)
    do = random_dout(q.shape, "bf16", seed=32, device="cuda")
    out, m, l = attn_fwd_stats(q, k, v, causal=True, scale=scale)
    dq, dk, dv = attn_bwd(q, k, v, out, do, m, l, causal=True, scale=scale)
    torch.cuda.synchronize()
    for b, h in HEADS:
        want = oracle.attention_backward_head(_np(q[b, h]), _np(k[b, h]), _np(v[b, h]),
                                              _np(do[b, h]), True, scale)
        for name, got, w in zip(("dQ", "dK", "dV"), (dq[b, h], dk[b, h], dv[b, h]), want):
            rel = float(np.max(np.abs(_np(got) - w)) / np.max(np.abs(w)))
            assert rel <= 2.0 ** -5, f"{name} head ({b},{h}): max err / max |ref| {rel}"
    del do, out, m, l, dq, dk, dv


def test_forward_f32_last_heads():
    q, k, v = random_qkv(B, H, N, N, D, "f32", seed=33, device="cuda")
    assert q.numel() > 2 ** 31
    scale = default_scale(D)
    out = attn_fwd(q, k, v, causal=False, scale=scale)
    torch.cuda.synchronize()
    for b, h in HEADS:
        want, _, _ = oracle.attention_rows(_np(q[b, h]), _np(k[b, h]), _np(v[b, h]), False, scale)
        err = float(np.max(np.abs(_np(out[b, h]) - want)))
        assert err <= TOL["f32"], f"head ({b},{h}): max abs err {err}"
    del q, k, v, out
    torch.cuda.empty_cache()
