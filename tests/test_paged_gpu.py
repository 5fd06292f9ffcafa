"""GPU parity of attention over a paged K/V cache (attn_decode_paged).

Each case calls the HIP library through the C ABI and compares every output
element with oracle.attention_paged (the plain definition on keys gathered
page by page) on the same inputs, upcast exactly to FP64.  Tolerances are
the attention tolerances of the other parity tests (max abs error 1e-5 FP32,
2e-3 FP16, 1e-2 BF16; lse = m + log l within the type's unit roundoff).
Page tables are seeded permutations, so logical and physical page order
differ; unused entries are -1.
"""

import numpy as np
import pytest
import torch

import oracle
from online_softmax_streaming_amd.workloads import make_paged

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "f16": 2e-3, "bf16": 1e-2}
LSE_TOL = {"f32": 1e-5, "f16": 2.0 ** -11 + 1e-5, "bf16": 2.0 ** -8 + 1e-5}


@pytest.fixture(scope="module")
def lib():
    import online_softmax_streaming_amd as m
    return m


def _np(t):
    return t.cpu().double().numpy() if t.is_floating_point() else t.cpu().numpy()


def _check(lib, inputs, causal, window, dtype, batches=None):
    q, kc, vc, table, lens = inputs
    scale = lib.default_scale(q.shape[-1])
    out, m, l = lib.attn_decode_paged(q, kc, vc, table, lens, causal=causal, window=window,
                                      want_stats=True)
    torch.cuda.synchronize()
    batches = range(q.shape[0]) if batches is None else batches
    for b in batches:
        want, wm, wl = oracle.attention_paged(_np(q)[b:b + 1], _np(kc), _np(vc), _np(table)[b:b + 1],
                                              _np(lens)[b:b + 1], causal, scale, window=window)
        got = _np(out)[b:b + 1]
        err = float(np.max(np.abs(got - want)))
        assert err <= TOL[dtype], (b, err)
        with np.errstate(divide="ignore"):
            lse = _np(m)[b:b + 1] + np.log(_np(l)[b:b + 1])
            wlse = wm + np.log(wl)
        fin = np.isfinite(wlse)
        assert np.array_equal(np.isfinite(lse), fin)
        assert np.max(np.abs(lse[fin] - wlse[fin]), initial=0.0) <= LSE_TOL[dtype]


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("h,hkv,nq,d,page,lens", [
    (8, 2, 1, 128, 16, [0, 37, 300, 1024]),
    (4, 4, 4, 64, 64, [2, 5, 130, 700]),    # causal: a sequence shorter than Nq
    (2, 1, 2, 32, 1, [1, 17, 64]),
    (4, 2, 8, 16, 32, [9, 200]),
    # Grouped heads on the matrix-core path: pages of 64 and 256 keys (one
    # page per 64-key tile or several tiles per page), 8-key pages (eight
    # pages per tile), 32 packed rows, and 2-key pages at D = 64 (below the
    # 8 rows of one load: the row-streaming path).
    (16, 2, 1, 128, 64, [1, 63, 64, 65, 2000]),
    (32, 1, 1, 64, 256, [300, 1, 1025]),
    (8, 2, 4, 128, 8, [4, 5, 77, 1500]),
    (12, 3, 8, 32, 16, [8, 9, 700]),
    (8, 4, 1, 64, 2, [3, 130]),
    (8, 2, 4, 64, 16, [2, 3, 600]),         # causal: rows that see no key at all
    (64, 1, 1, 128, 16, [1, 777, 3000]),    # one K/V head for 64 query heads: two row chunks
    (16, 2, 5, 64, 8, [5, 300]),            # 40 rows per K/V head
    (16, 2, 1, 128, 1, [1, 100, 3000]),     # one-key pages: per-row addresses
    (8, 2, 3, 32, 4, [7, 1000]),            # pages below the 16 rows of one load
    # D = 16: one 16-byte load moves 32 key rows; pages of 1 and 4 keys take
    # per-row addresses (two loads of 32 rows per tile), 16-key pages too
    # (below the 32 rows of one load), 32-key pages the descriptor path.
    (8, 2, 1, 16, 1, [1, 40, 1300]),
    (8, 2, 2, 16, 4, [3, 65, 999]),
    (16, 4, 1, 16, 16, [2, 17, 2048]),
    (4, 1, 4, 16, 32, [1, 100, 700]),
])
def test_parity(lib, dtype, causal, h, hkv, nq, d, page, lens):
    inputs = make_paged(len(lens), h, hkv, nq, d, page, lens, dtype, seed=h + nq + d + page,
                        device="cuda", share_first_page=True)
    _check(lib, inputs, causal, 0, dtype)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("window,nq", [(1, 1), (100, 1), (256, 1), (40, 8), (3, 4)])
def test_sliding_window(lib, dtype, window, nq):
    inputs = make_paged(3, 4, 2, nq, 128, 16, [1000, 4096, 50], dtype, seed=window + nq,
                        device="cuda")
    _check(lib, inputs, True, window, dtype)


@pytest.mark.parametrize("window,nq,page", [(64, 1, 64), (65, 2, 32), (1000, 4, 16), (5000, 1, 128),
                                           (100, 2, 1)])
def test_sliding_window_grouped(lib, window, nq, page):
    # Eight query heads per K/V head: the splits start at the window's lower
    # bound rounded down to a 64-key tile.
    inputs = make_paged(3, 16, 2, nq, 128, page, [1000, 4096, 50], "bf16", seed=window + page,
                        device="cuda")
    _check(lib, inputs, True, window, "bf16")


def test_window_one_returns_the_last_value(lib):
    q, kc, vc, table, lens = make_paged(2, 2, 2, 1, 64, 16, [33, 100], "bf16", seed=3, device="cuda")
    out, _, l = lib.attn_decode_paged(q, kc, vc, table, lens, causal=True, window=1, want_stats=True)
    torch.cuda.synchronize()
    for b, n in enumerate((33, 100)):
        j = n - 1
        page = int(table[b, j // 16])
        assert torch.equal(out[b, :, 0], vc[page, :, j % 16])
        assert torch.all(l[b] == 1.0)


def test_absent_pages_contribute_nothing(lib):
    # A table entry outside the cache is an absent key; noncausal attention
    # does not depend on key positions, so the oracle drops those keys.
    q, kc, vc, table, lens = make_paged(1, 2, 2, 1, 64, 16, [64], "f16", seed=4, device="cuda")
    bad = table.clone()
    bad[0, 1] = 1 << 20
    bad[0, 2] = -7
    out, _, _ = lib.attn_decode_paged(q, kc, vc, bad, lens, causal=False)
    torch.cuda.synchronize()
    keep = [0, 3]
    k = np.concatenate([_np(kc)[int(table[0, p])] for p in keep], axis=1)  # [Hkv, 32, D]
    v = np.concatenate([_np(vc)[int(table[0, p])] for p in keep], axis=1)
    scale = lib.default_scale(64)
    for h in range(2):
        want, _, _ = oracle.attention_rows(_np(q)[0, h], k[h], v[h], False, scale)
        assert np.max(np.abs(_np(out)[0, h] - want)) <= TOL["f16"]


@pytest.mark.parametrize("page,d", [(2, 64), (16, 64), (64, 64), (1, 16), (4, 16), (16, 16)])
def test_absent_pages_contribute_nothing_grouped(lib, page, d):
    # Grouped heads (four query heads per K/V head, two query rows): an
    # absent page inside a 64-key tile (pages of 1 to 16 keys) or a whole
    # absent tile (page 64) masks exactly its keys; at D = 16 the per-row
    # path moves 32 rows per load.
    npg = 4
    q, kc, vc, table, lens = make_paged(1, 8, 2, 2, d, page, [npg * page], "bf16", seed=14,
                                        device="cuda")
    bad = table.clone()
    bad[0, 1] = 1 << 20
    bad[0, 2] = -7
    out, _, _ = lib.attn_decode_paged(q, kc, vc, bad, lens, causal=False)
    torch.cuda.synchronize()
    keep = [0, 3]
    k = np.concatenate([_np(kc)[int(table[0, p])] for p in keep], axis=1)
    v = np.concatenate([_np(vc)[int(table[0, p])] for p in keep], axis=1)
    scale = lib.default_scale(d)
    for h in range(8):
        want, _, _ = oracle.attention_rows(_np(q)[0, h], k[h // 4], v[h // 4], False, scale)
        assert np.max(np.abs(_np(out)[0, h] - want)) <= TOL["bf16"], h


def test_window_one_returns_the_last_value_grouped(lib):
    # One visible key per row: weight exactly 1 on the matrix-core path too.
    q, kc, vc, table, lens = make_paged(2, 8, 2, 1, 128, 16, [33, 3000], "bf16", seed=15,
                                        device="cuda")
    out, _, l = lib.attn_decode_paged(q, kc, vc, table, lens, causal=True, window=1, want_stats=True)
    torch.cuda.synchronize()
    for b, n in enumerate((33, 3000)):
        j = n - 1
        page = int(table[b, j // 16])
        for h in range(8):
            assert torch.equal(out[b, h, 0], vc[page, h // 4, j % 16]), (b, h)
        assert torch.all(l[b] == 1.0)


def test_unused_table_entries_are_not_read(lib):
    inputs = make_paged(2, 2, 1, 1, 64, 16, [20, 200], "bf16", seed=5, device="cuda")
    q, kc, vc, table, lens = inputs
    assert int(table[0, 5]) == -1  # past sequence 0's two pages
    _check(lib, inputs, True, 0, "bf16")


def test_serving_shape_sampled(lib):
    # Serving-sized decode: 16 sequences of mixed length up to 8192 keys,
    # 32 query heads over 8 K/V heads, 16-key pages; two sequences checked.
    rng = np.random.default_rng(0)
    lens = [int(x) for x in rng.integers(1, 8193, size=16)]
    inputs = make_paged(16, 32, 8, 1, 128, 16, lens, "bf16", seed=6, device="cuda")
    _check(lib, inputs, True, 0, "bf16", batches=[0, 15])


def test_bench_shape_grouped_sampled(lib):
    # The paged grouped decode the benchmark times, in its launch
    # configuration: B16 H32 Hkv4 Nq1, 32768 keys per sequence in shuffled
    # 16-key pages, D128 bf16, causal; two sequences checked.  The oracle gets
    # the pages of the checked sequence only (same table order), which is all
    # it reads.
    q, kc, vc, table, lens = make_paged(16, 32, 4, 1, 128, 16, [32768] * 16, "bf16", seed=2,
                                        device="cuda")
    scale = lib.default_scale(128)
    out, m, l = lib.attn_decode_paged(q, kc, vc, table, lens, causal=True, scale=scale,
                                      want_stats=True)
    torch.cuda.synchronize()
    npg = 32768 // 16
    for b in (0, 15):
        pages = table[b, :npg].long()
        ksub, vsub = _np(kc[pages]), _np(vc[pages])
        tsub = np.arange(npg, dtype=np.int32).reshape(1, npg)
        want, wm, wl = oracle.attention_paged(_np(q)[b:b + 1], ksub, vsub, tsub, _np(lens)[b:b + 1],
                                              True, scale)
        err = float(np.max(np.abs(_np(out)[b:b + 1] - want)))
        assert err <= TOL["bf16"], (b, err)
        lse = _np(m)[b:b + 1] + np.log(_np(l)[b:b + 1])
        assert np.max(np.abs(lse - (wm + np.log(wl)))) <= LSE_TOL["bf16"], b
