"""GPU parity of attention over packed variable-length sequences
(attn_fwd_varlen).

Every case calls the HIP library through the C ABI and compares each output
element with oracle.attention_varlen on the same inputs, upcast exactly to
FP64, with the attention tolerances of the other parity tests (max abs
error 1e-5 FP32, 2e-3 FP16, 1e-2 BF16; lse = m + log l within the type's unit
roundoff).  Equal-length batches must also equal attn_fwd_gqa on the
transposed layout bit for bit: the kernels do the same arithmetic with
different addressing.
"""

import numpy as np
import pytest
import torch

import oracle
from online_softmax_streaming_amd.workloads import make_varlen, random_qkv

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "f16": 2e-3, "bf16": 1e-2}
LSE_TOL = {"f32": 1e-5, "f16": 2.0 ** -11 + 1e-5, "bf16": 2.0 ** -8 + 1e-5}


@pytest.fixture(scope="module")
def lib():
    import online_softmax_streaming_amd as m
    return m


def _np(t):
    return t.cpu().double().numpy() if t.is_floating_point() else t.cpu().numpy()


def _check(lib, inputs, causal, dtype):
    q, k, v, cu_q, cu_k = inputs
    out, m, l = lib.attn_fwd_varlen(q, k, v, cu_q, cu_k, causal=causal, want_stats=True)
    torch.cuda.synchronize()
    scale = lib.default_scale(q.shape[-1])
    want, wm, wl = oracle.attention_varlen(_np(q), _np(k), _np(v), _np(cu_q), _np(cu_k), causal,
                                           scale)
    err = float(np.max(np.abs(_np(out) - want), initial=0.0))
    assert err <= TOL[dtype], err
    with np.errstate(divide="ignore"):
        lse = _np(m) + np.log(_np(l))
        wlse = wm + np.log(wl)
    fin = np.isfinite(wlse)
    assert np.array_equal(np.isfinite(lse), fin)
    assert np.max(np.abs(lse[fin] - wlse[fin]), initial=0.0) <= LSE_TOL[dtype]


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("h,hkv,d,lens_q,lens_k", [
    (4, 2, 128, [300, 0, 1, 77, 1024, 5], [300, 3, 1, 77, 1024, 40]),
    (2, 2, 64, [513, 9, 256], [100, 700, 256]),     # Nq != Nk in both directions
    (8, 1, 32, [64, 65, 257], [0, 65, 300]),        # a sequence with no keys
    (2, 1, 16, [700], [700]),
])
def test_parity(lib, dtype, causal, h, hkv, d, lens_q, lens_k):
    inputs = make_varlen(lens_q, lens_k, h, hkv, d, dtype, seed=sum(lens_q) + d, device="cuda")
    _check(lib, inputs, causal, dtype)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("nseq", [40, 90])
def test_many_sequences_of_mixed_lengths(lib, causal, nseq):
    # 40 sequences: workgroups take them in decreasing key count (ranked in
    # LDS, ties included); 90: beyond the ranking's 64, input order.
    g = np.random.default_rng(nseq)
    lens = [int(x) for x in g.integers(1, 700, size=nseq)]
    lens[3] = lens[7] = lens[11] = 333  # ties in the ranking
    inputs = make_varlen(lens, lens, 4, 2, 64, "bf16", seed=nseq, device="cuda")
    _check(lib, inputs, causal, "bf16")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("causal", [False, True])
def test_equal_lengths_equal_batched_kernel(lib, dtype, causal):
    # 32 x 4 heads: the batched call then takes the same tiled kernel as the
    # varlen one (small problems split keys over waves instead).
    b, h, hkv, n, d = 32, 4, 2, 300, 128
    q, _, _ = random_qkv(b, h, n, n, d, dtype, seed=1, device="cuda")
    _, k, v = random_qkv(b, hkv, n, n, d, dtype, seed=2, device="cuda")
    out, m, l = lib.attn_fwd_gqa(q, k, v, causal=causal, want_stats=True)
    qp = q.transpose(1, 2).reshape(b * n, h, d).contiguous()
    kp = k.transpose(1, 2).reshape(b * n, hkv, d).contiguous()
    vp = v.transpose(1, 2).reshape(b * n, hkv, d).contiguous()
    cu = torch.arange(0, (b + 1) * n, n, dtype=torch.int32, device="cuda")
    outp, mp, lp = lib.attn_fwd_varlen(qp, kp, vp, cu, cu, max_seqlen_q=n, causal=causal,
                                       want_stats=True)
    torch.cuda.synchronize()
    assert torch.equal(outp, out.transpose(1, 2).reshape(b * n, h, d))
    assert torch.equal(mp, m.permute(1, 0, 2).reshape(h, b * n))
    assert torch.equal(lp, l.permute(1, 0, 2).reshape(h, b * n))


def test_max_seqlen_from_offsets(lib):
    inputs = make_varlen([5, 40, 17], [5, 40, 17], 2, 2, 64, "bf16", seed=3, device="cuda")
    q, k, v, cu_q, cu_k = inputs
    a, _, _ = lib.attn_fwd_varlen(q, k, v, cu_q, cu_k, causal=True)
    b, _, _ = lib.attn_fwd_varlen(q, k, v, cu_q, cu_k, max_seqlen_q=40, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_many_short_sequences(lib):
    rng = np.random.default_rng(0)
    lens = [int(x) for x in rng.integers(1, 300, size=40)]
    inputs = make_varlen(lens, lens, 4, 1, 64, "f16", seed=4, device="cuda")
    _check(lib, inputs, True, "f16")


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("h,hkv,d,lens_q,lens_k", [
    (4, 2, 128, [512], [8192]),                 # one chunk over a long context: 8 splits
    (4, 1, 64, [300, 100], [5000, 2000]),       # the shorter sequence's late splits are empty
    (2, 2, 128, [200, 0, 50], [6000, 3000, 0]),  # no rows; no keys
    (2, 1, 32, [64], [16384]),
])
def test_split_kv(lib, dtype, causal, h, hkv, d, lens_q, lens_k):
    # Few query tiles over many keys: each tile's keys are split over
    # workgroups (the plan takes total_k as the longest sequence's key
    # count) and the partial states combined per sequence.
    inputs = make_varlen(lens_q, lens_k, h, hkv, d, dtype, seed=sum(lens_k) + d, device="cuda")
    _check(lib, inputs, causal, dtype)


@pytest.mark.parametrize("causal", [False, True])
def test_split_kv_longer_sequence_never_wrong(lib, causal):
    # max_seqlen_q = 256 with a 300-row sequence: the rows of that sequence
    # past the query tiles the grid holds are left as they were (noncausal:
    # rows 256..; causal, tiles aligned to the last row: rows 44..), every
    # other row matches the oracle, and no row is written wrong.
    q, k, v, cu_q, cu_k = make_varlen([300, 40], [9000, 3000], 4, 4, 64, "bf16", seed=11,
                                      device="cuda")
    out = torch.full_like(q, 7.0)
    lib.attn_fwd_varlen(q, k, v, cu_q, cu_k, max_seqlen_q=256, causal=causal, out=out)
    torch.cuda.synchronize()
    scale = lib.default_scale(64)
    want, _, _ = oracle.attention_varlen(_np(q), _np(k), _np(v), _np(cu_q), _np(cu_k), causal,
                                         scale)
    got = _np(out)
    skipped = np.zeros(got.shape[0], dtype=bool)
    skipped[(44 if causal else 256):300] = True
    assert np.all(got[skipped] == 7.0)
    assert float(np.max(np.abs(got[~skipped] - want[~skipped]))) <= TOL["bf16"]
