"""GPU parity of grouped-query attention (attn_fwd_gqa).

K and V carry Hkv heads and query head h reads K/V head h // (H // Hkv).
The oracle is the plain definition applied to K/V with each head repeated
H // Hkv times (oracle.attention on the expanded tensors).  Tolerances are
the attention tolerances of the other parity tests.  The same kernels run
with only the K/V head index changed, so the grouped call must also equal,
bit for bit, attn_fwd on explicitly repeated K/V.
"""

import numpy as np
import pytest
import torch

import oracle
from online_softmax_streaming_amd.workloads import random_qkv

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "f16": 2e-3, "bf16": 1e-2}
LSE_TOL = {"f32": 1e-5, "f16": 2.0 ** -11 + 1e-5, "bf16": 2.0 ** -8 + 1e-5}


@pytest.fixture(scope="module")
def lib():
    import online_softmax_streaming_amd as m
    return m


def _grouped(b, h, hkv, nq, nk, d, dtype, seed):
    q, _, _ = random_qkv(b, h, nq, nk, d, dtype, seed=seed, device="cuda")
    _, k, v = random_qkv(b, hkv, nq, nk, d, dtype, seed=seed + 1, device="cuda", k_ramp=0.01)
    return q, k, v


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("h,hkv,nq,nk,d", [
    (8, 1, 300, 300, 64), (8, 2, 259, 517, 128), (8, 4, 517, 259, 64), (6, 3, 1, 1000, 128),
    (8, 2, 5, 700, 64), (4, 4, 129, 129, 32),
    # decode with grouped heads: G * Nq rows of a K/V head share one matrix
    # tile (up to 32), several key splits, ragged and causal key ends
    (32, 8, 4, 5000, 128), (16, 1, 2, 3001, 64), (32, 1, 1, 2049, 32), (8, 2, 3, 4099, 16),
    (12, 3, 8, 777, 128),
    # fewer keys than query rows (causal: rows 0 .. Nq - Nk - 1 see no key),
    # and a single key
    (8, 2, 6, 2, 64), (16, 2, 2, 1, 128),
    # more than 32 rows per K/V head: chunks of 32 rows, each reading the
    # K/V tiles once (MQA with 64 query heads; 64 and 96 packed rows; 40
    # rows, the second chunk ragged)
    (64, 1, 1, 3001, 128), (16, 2, 8, 700, 64), (48, 1, 2, 999, 32), (8, 1, 5, 1500, 64),
])
def test_parity(lib, dtype, causal, h, hkv, nq, nk, d):
    q, k, v = _grouped(2, h, hkv, nq, nk, d, dtype, seed=h * 10 + hkv + nq)
    out, m, l = lib.attn_fwd_gqa(q, k, v, causal=causal, want_stats=True)
    torch.cuda.synchronize()
    g = h // hkv
    qd = q.cpu().double().numpy()
    kd = np.repeat(k.cpu().double().numpy(), g, axis=1)
    vd = np.repeat(v.cpu().double().numpy(), g, axis=1)
    scale = lib.default_scale(d)
    want, wm, wl = oracle.attention(qd, kd, vd, causal, scale)
    err = np.max(np.abs(out.cpu().double().numpy() - want))
    assert err <= TOL[dtype], err
    with np.errstate(divide="ignore"):  # rows with no visible key: l = 0, lse = -inf
        lse = m.cpu().double().numpy() + np.log(l.cpu().double().numpy())
        wlse = wm + np.log(wl)
    fin = np.isfinite(wlse)
    assert np.array_equal(np.isfinite(lse), fin)
    assert np.max(np.abs(lse[fin] - wlse[fin]), initial=0.0) <= LSE_TOL[dtype]


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("h,hkv,nq,nk,d", [
    (8, 2, 16, 9000, 64), (6, 3, 20, 8192, 32),  # 64 / 40 rows per K/V head: decode route
    (8, 2, 17, 8192, 128),                       # 68 rows per K/V head: prefill kernels
])
def test_decode_route_mid_rows(lib, dtype, causal, h, hkv, nq, nk, d):
    # 9..32 query rows per head with at most 64 per K/V head over >= 8192
    # keys take the split-key path on the matrix cores (bf16/f16 only, so
    # FP32 is not a case here; with these inputs' ramped keys the logits reach
    # ~130 in base 2, beyond what FP32 scores carry to 1e-5).
    test_parity(lib, dtype, causal, h, hkv, nq, nk, d)


@pytest.mark.parametrize("dtype,causal,h,hkv,nq,nk,d", [
    ("bf16", True, 8, 2, 256, 8192, 128), ("f16", False, 4, 1, 300, 12000, 64)])
def test_split_kv_grouped(lib, dtype, causal, h, hkv, nq, nk, d):
    # Few query tiles over many keys with grouped K/V heads: each tile's keys
    # split over workgroups (8 and 11 splits), partial states combined.
    test_parity(lib, dtype, causal, h, hkv, nq, nk, d)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("nq", [1, 300])
def test_equals_mha_on_repeated_kv(lib, dtype, nq):
    q, k, v = _grouped(2, 8, 2, nq, 640, 128, dtype, seed=77)
    got = lib.attn_fwd_gqa(q, k, v, causal=True)[0]
    kr = k.repeat_interleave(4, dim=1).contiguous()
    vr = v.repeat_interleave(4, dim=1).contiguous()
    want = lib.attn_fwd(q, kr, vr, causal=True)
    torch.cuda.synchronize()
    if nq == 1 and dtype != "f32":
        # A grouped decode packs the group's rows into one matrix tile (each
        # K/V tile read once); the repeated-head call streams rows one by
        # one.  Both are checked against the oracle in test_parity.
        assert float((got.float() - want.float()).abs().max()) <= TOL[dtype]
    else:
        assert torch.equal(got, want)


def test_hkv_equal_h_is_attn_fwd_stats(lib):
    q, k, v = random_qkv(1, 4, 200, 333, 64, "f16", seed=3, device="cuda")
    a, am, al = lib.attn_fwd_gqa(q, k, v, causal=True, want_stats=True)
    b, bm, bl = lib.attn_fwd_stats(q, k, v, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(am, bm) and torch.equal(al, bl)


def test_bench_shape_sampled(lib):
    # The grouped decode the benchmark times, in its launch configuration:
    # B16 H32 Hkv4 Nq1 Nk32768 D128 bf16, contiguous K/V, noncausal, inputs
    # drawn as the benchmark draws them; three (b, h) rows checked.
    b_, h_, hkv, nk, d = 16, 32, 4, 32768, 128
    q, _, _ = random_qkv(b_, h_, 1, 1, d, "bf16", seed=0, device="cuda")
    _, k, v = random_qkv(b_, hkv, 1, nk, d, "bf16", seed=1, device="cuda")
    scale = lib.default_scale(d)
    out, m, l = lib.attn_fwd_gqa(q, k, v, scale=scale, want_stats=True)
    torch.cuda.synchronize()

    def np64(t):
        return t.cpu().double().numpy()

    for bb, hh in ((0, 0), (7, 13), (15, 31)):
        hk = hh // (h_ // hkv)
        want, wm, wl = oracle.attention_rows(np64(q[bb, hh]), np64(k[bb, hk]), np64(v[bb, hk]), False,
                                             scale)
        err = float(np.max(np.abs(np64(out[bb, hh]) - want)))
        assert err <= TOL["bf16"], ((bb, hh), err)
        lse = np64(m[bb, hh]) + np.log(np64(l[bb, hh]))
        assert np.max(np.abs(lse - (wm + np.log(wl)))) <= LSE_TOL["bf16"], (bb, hh)


def test_bench_shape_nq4_sampled(lib):
    # The multi-row decode the benchmark times: plain heads (B16 H32 Hkv32)
    # with 4 causal query rows each over 32768 keys, D128 bf16, inputs drawn
    # as the benchmark draws them; two heads checked.
    b_, h_, nq, nk, d = 16, 32, 4, 32768, 128
    q, _, _ = random_qkv(b_, h_, nq, 1, d, "bf16", seed=0, device="cuda")
    _, k, v = random_qkv(b_, h_, 1, nk, d, "bf16", seed=1, device="cuda")
    scale = lib.default_scale(d)
    out, m, l = lib.attn_fwd_gqa(q, k, v, causal=True, scale=scale, want_stats=True)
    torch.cuda.synchronize()

    def np64(t):
        return t.cpu().double().numpy()

    for bb, hh in ((0, 0), (15, 31)):
        want, wm, wl = oracle.attention_rows(np64(q[bb, hh]), np64(k[bb, hh]), np64(v[bb, hh]), True,
                                             scale)
        err = float(np.max(np.abs(np64(out[bb, hh]) - want)))
        assert err <= TOL["bf16"], ((bb, hh), err)
        lse = np64(m[bb, hh]) + np.log(np64(l[bb, hh]))
        assert np.max(np.abs(lse - (wm + np.log(wl)))) <= LSE_TOL["bf16"], (bb, hh)
    del q, k, v, out
    torch.cuda.empty_cache()
