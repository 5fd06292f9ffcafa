"""attn_fwd and attn_fwd_stats under HIP graph capture.

Most shapes here take the tiled prefill kernels, which allocate nothing and
launch only kernels on the caller's stream.  Two take the paths with
partial states: the split-KV prefill (few query tiles over many keys) and
the split-key decode (few rows); under capture each such call takes its own
hipMallocAsync / hipFreeAsync pair, which the graph records as allocation
nodes (outside capture they use the stream's cached scratch).  Each test
captures calls once, replays the graph several times with eager work and
synchronisations between the replays, and checks every replay bit for bit
against an eager call on the same inputs (the kernels are deterministic),
including after the captured input buffers were refilled in place.  The
eager result itself is checked against the FP64 oracle on one small case.
"""

import numpy as np
import pytest
import torch

import oracle
from online_softmax_streaming_amd import attn_fwd, attn_fwd_stats, default_scale
from online_softmax_streaming_amd.workloads import random_qkv

pytestmark = pytest.mark.gpu


def _capture(fn):
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()  # first call outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


@pytest.mark.parametrize("dtype,d,causal,nq,nk", [
    ("bf16", 128, True, 300, 300),
    ("f16", 64, False, 77, 533),
    ("f32", 64, True, 130, 130),
    # Paths with stream-ordered scratch (allocation nodes in the graph): the
    # split-KV prefill (8 key splits) and the split-key decode.
    ("bf16", 128, True, 256, 8192),
    ("f16", 64, False, 4, 3000),
])
def test_replay_matches_eager(dtype, d, causal, nq, nk):
    q, k, v = random_qkv(2, 3, nq, nk, d, dtype, seed=nq + nk, device="cuda")
    scale = default_scale(d)
    out = torch.full_like(q, 7.0)
    g = _capture(lambda: attn_fwd(q, k, v, causal=causal, scale=scale, out=out))
    for rep in range(4):
        # Fresh inputs written in place into the captured buffers.
        nq_, nk_, nv_ = random_qkv(2, 3, nq, nk, d, dtype, seed=100 + rep, device="cuda")
        q.copy_(nq_)
        k.copy_(nk_)
        v.copy_(nv_)
        out.fill_(-3.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        want = attn_fwd(q, k, v, causal=causal, scale=scale)
        torch.cuda.synchronize()
        assert torch.equal(out, want), f"replay {rep}"


def test_replay_row_states_and_oracle():
    q, k, v = random_qkv(1, 2, 200, 200, 64, "bf16", seed=3, device="cuda")
    scale = default_scale(64)
    out = torch.empty_like(q)
    m = torch.empty((1, 2, 200), dtype=torch.float32, device="cuda")
    l = torch.empty_like(m)

    def call():
        attn_fwd_stats(q, k, v, causal=True, scale=scale, out=out, m_out=m, l_out=l)

    g = _capture(call)
    eo, em, el = attn_fwd_stats(q, k, v, causal=True, scale=scale)
    torch.cuda.synchronize()
    for rep in range(3):
        out.zero_()
        m.zero_()
        l.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eo) and torch.equal(m, em) and torch.equal(l, el), f"replay {rep}"
    want, _, _ = oracle.attention(*(t.cpu().double().numpy() for t in (q, k, v)), True, scale)
    assert float(np.max(np.abs(out.cpu().double().numpy() - want))) <= 1e-2
