"""The per-stream scratch of the partial-state paths (split-key decode,
split-KV prefill, backward, wide-row softmax): one buffer per stream, reused
across calls of different sizes, and separate buffers on separate streams.

Results must not depend on what an earlier call left in the buffer: every
call below is repeated after calls of other sizes (on the same stream, and
interleaved with calls on a second stream without synchronising between
them) and compared bit for bit with its first result.
"""

import pytest
import torch

from online_softmax_streaming_amd import attn_bwd, attn_fwd, attn_fwd_stats, default_scale
from online_softmax_streaming_amd.workloads import random_qkv

pytestmark = pytest.mark.gpu

DEV = "cuda:0"

# (B, H, Nq, Nk, D, causal, dtype): split-key decode (small and large
# scratch), split-KV prefill (4 and 8 key splits).
CASES = [
    (1, 4, 1, 3000, 64, False, "bf16"),
    (8, 32, 4, 20000, 128, True, "bf16"),
    (1, 32, 512, 8192, 128, True, "bf16"),
    (1, 2, 256, 16384, 32, True, "f16"),
]


def _inputs():
    return [random_qkv(b, h, nq, nk, d, dt, seed=i, device=DEV, k_ramp=0.002)
            for i, (b, h, nq, nk, d, _, dt) in enumerate(CASES)]


def _run(qkv, case):
    q, k, v = qkv
    return attn_fwd(q, k, v, causal=case[5], scale=default_scale(case[4]))


def test_reuse_across_sizes_on_one_stream():
    print("[scratch] one stream, sizes small -> large -> small", flush=True)
    inp = _inputs()
    first = [_run(x, c) for x, c in zip(inp, CASES)]
    torch.cuda.synchronize()
    # Largest first, then the rest in reverse: every call now finds the
    # buffer holding another call's partial states.
    order = [1, 2, 3, 0, 2, 1, 0, 3]
    again = [(i, _run(inp[i], CASES[i])) for i in order]
    torch.cuda.synchronize()
    for i, out in again:
        assert torch.equal(out, first[i]), f"case {CASES[i]} changed after reuse"


def test_two_streams_interleaved():
    print("[scratch] two streams, no synchronisation between them", flush=True)
    inp = _inputs()
    want = [_run(x, c) for x, c in zip(inp, CASES)]
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    outs = []
    for rep in range(3):
        for i in range(len(CASES)):
            s = s1 if (i + rep) % 2 == 0 else s2
            with torch.cuda.stream(s):
                outs.append((i, _run(inp[i], CASES[i])))
    torch.cuda.synchronize()
    for i, out in outs:
        assert torch.equal(out, want[i]), f"case {CASES[i]} differs on a side stream"


def test_backward_after_forward_scratch():
    # The backward's (lse, Delta) scratch shares the stream's buffer with the
    # forward paths: its gradients must not change after a split-KV forward
    # has filled the buffer with its partial states.
    print("[scratch] backward after split-KV forward", flush=True)
    q, k, v = random_qkv(1, 4, 512, 4096, 64, "bf16", seed=5, device=DEV)
    dout = torch.randn_like(q)
    scale = default_scale(64)
    out, m, l = attn_fwd_stats(q, k, v, causal=True, scale=scale)
    torch.cuda.synchronize()
    grads = attn_bwd(q, k, v, out, dout, m, l, causal=True, scale=scale)
    big = random_qkv(*CASES[2][:5], CASES[2][6], seed=2, device=DEV)
    _run(big, CASES[2])  # fills the buffer with other partial states
    again = attn_bwd(q, k, v, out, dout, m, l, causal=True, scale=scale)
    torch.cuda.synchronize()
    for a, b in zip(grads, again):
        assert torch.equal(a, b)
