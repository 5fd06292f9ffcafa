"""attn_decode_paged_noalloc: the paged decode entry point that allocates
nothing, for callers that cannot allocate (graph capture, serving loops).

Each GPU case calls the new entry point through the C ABI and compares its
output with attn_decode_paged (the existing entry point, itself checked
against the FP64 oracle in test_paged_gpu.py) on the same inputs: bit for bit
when the usual split plan fits the fixed 4 MiB buffer, and within the
attention tolerances (max abs 1e-5 FP32, 2e-3 FP16, 1e-2 BF16) when fewer
splits are taken.  Two calls in a row, the second on a smaller problem, check
that the buffer's leftover contents from the first call never leak into the
second.  Oversized problems are rejected before any device work.
"""

import numpy as np
import pytest
import torch

import oracle
from online_softmax_streaming_amd.workloads import make_paged

TOL = {"f32": 1e-5, "f16": 2e-3, "bf16": 1e-2}
FIXED_BYTES = 4 << 20


@pytest.fixture(scope="module")
def lib():
    import online_softmax_streaming_amd as m
    return m


def _both(lib, inputs, causal, window=0):
    q, kc, vc, table, lens = inputs
    want, wm, wl = lib.attn_decode_paged(q, kc, vc, table, lens, causal=causal, window=window,
                                         want_stats=True)
    got, gm, gl = lib.attn_decode_paged_noalloc(q, kc, vc, table, lens, causal=causal,
                                                window=window, want_stats=True)
    torch.cuda.synchronize()
    return (got, gm, gl), (want, wm, wl)


@pytest.mark.gpu
@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
def test_two_calls_in_a_row_equal_the_allocating_entry_point(lib, dtype):
    # First call: 4 sequences of up to 3000 keys, grouped heads (bf16/f16:
    # the matrix-core partial kernel; f32: the row-streaming kernel).
    # Second call: a smaller problem (fewer rows, fewer splits), so the
    # buffer still holds the first call's partial states in slots the
    # second call does not use.
    first = make_paged(4, 8, 2, 2, 128, 16, [3000, 1, 777, 2048], dtype, seed=1, device="cuda")
    (g1, gm1, gl1), (w1, wm1, wl1) = _both(lib, first, causal=True)
    second = make_paged(2, 4, 4, 1, 64, 32, [5, 400], dtype, seed=2, device="cuda")
    (g2, gm2, gl2), (w2, wm2, wl2) = _both(lib, second, causal=False)
    for got, want in ((g1, w1), (gm1, wm1), (gl1, wl1), (g2, w2), (gm2, wm2), (gl2, wl2)):
        assert torch.equal(got, want)
    # The smaller call also against the oracle directly.
    q, kc, vc, table, lens = (t.cpu() for t in second)
    scale = lib.default_scale(64)
    ref, _, _ = oracle.attention_paged(q.double().numpy(), kc.double().numpy(),
                                       vc.double().numpy(), table.numpy(), lens.numpy(), False,
                                       scale)
    assert float(np.max(np.abs(g2.cpu().double().numpy() - ref))) <= TOL[dtype]


@pytest.mark.gpu
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_capped_plan_stays_within_tolerance(lib, dtype):
    # One sequence of 32768 keys, 32 query heads on 4 K/V heads, 4 rows per
    # head at D = 128: 32 packed rows per K/V head on the matrix-core path,
    # whose usual plan takes 64 key splits of 512 keys, i.e. 128 rows x 64
    # splits x 130 FP32 values = 4.26 MB of partial states, more than the
    # fixed 4 MiB.  The call takes 63 splits instead.  Then a second,
    # smaller call in a row, which fits and must match bit for bit.
    rows, usual_splits, d = 1 * 32 * 4, 64, 128
    assert rows * usual_splits * (d + 2) * 4 > FIXED_BYTES
    big = make_paged(1, 32, 4, 4, d, 64, [32768], dtype, seed=3, device="cuda", spare_pages=0)
    (g, gm, gl), (w, wm, wl) = _both(lib, big, causal=True)
    assert torch.isfinite(g).all()
    assert float((g.double() - w.double()).abs().max()) <= TOL[dtype]
    lse_g = gm.double() + gl.double().log()
    lse_w = wm.double() + wl.double().log()
    assert float((lse_g - lse_w).abs().max()) <= {"bf16": 2.0 ** -8, "f16": 2.0 ** -11}[dtype] + 1e-5
    small = make_paged(3, 8, 8, 1, 128, 16, [1000, 17, 3], dtype, seed=4, device="cuda")
    (g2, _, _), (w2, _, _) = _both(lib, small, causal=False)
    assert torch.equal(g2, w2)


@pytest.mark.gpu
def test_graph_capture_replays_match_eager(lib):
    # The caller this entry point is for: a decode step captured once into a
    # HIP graph and replayed, with eager work and synchronisations between
    # replays; every replay must equal an eager call.
    q, kc, vc, table, lens = make_paged(4, 16, 4, 1, 128, 16, [4000, 100, 2500, 1], "bf16",
                                        seed=5, device="cuda")
    out = torch.empty_like(q)
    m = torch.empty(q.shape[:3], dtype=torch.float32, device="cuda")
    l = torch.empty_like(m)

    def call():
        lib.attn_decode_paged_noalloc(q, kc, vc, table, lens, causal=True, out=out, m_out=m,
                                      l_out=l, want_stats=True)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()  # first call (device buffer lookup) outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    torch.cuda.synchronize()
    want, wm, wl = lib.attn_decode_paged(q, kc, vc, table, lens, causal=True, want_stats=True)
    torch.cuda.synchronize()
    for rep in range(4):
        out.fill_(-5.0)
        m.zero_()
        # Eager work on the same buffer between replays.
        lib.attn_decode_paged_noalloc(q[:2], kc, vc, table[:2], lens[:2], causal=False)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, want) and torch.equal(m, wm) and torch.equal(l, wl), rep


def test_oversized_problem_is_rejected_before_device_work(lib):
    # B*H*Nq*(D+2)*4 > 4 MiB even with one split: rejected on the host, so
    # the fake (never dereferenced) pointers below are never used.
    import ctypes
    from online_softmax_streaming_amd import _lib
    b, h, nq, d = 512, 16, 1, 128
    assert b * h * nq * (d + 2) * 4 > FIXED_BYTES
    p = [ctypes.c_void_p(0x40000000 * (i + 1)) for i in range(6)]
    rc = _lib.lib().attn_decode_paged_noalloc(*p, b, h, h, nq, d, 8, 16, 4, 1, 0, 0.125,
                                              lib.ATTN_BF16, None, None, None)
    assert rc == lib.ATTN_E_UNSUPPORTED
    assert b"fixed buffer" in _lib.lib().attn_last_error()
    # Argument errors come first, as in attn_decode_paged.
    rc = _lib.lib().attn_decode_paged_noalloc(*p, b, h, h, nq, d, 8, 3, 4, 1, 0, 0.125,
                                              lib.ATTN_BF16, None, None, None)
    assert rc == lib.ATTN_E_INVALID
