"""GPU parity of attention with dropout (attn_fwd_dropout).

The kernels and the oracle each implement Philox4x64-10 from its published
definition (the oracle's is pinned bit for bit to numpy.random.Philox), so
the keep decisions must agree exactly: with Q = 0 every visible weight is 1
and V built from identity blocks makes each output element encode which
keys were kept.  Outputs are compared element by element with
oracle.attention_dropout on the same inputs, with the attention tolerances
of the other parity tests multiplied by the keep gain 65536 / (65536 - T)
(every kept weight is scaled by it).  p = 0 must equal attn_fwd_gqa bit for
bit.
"""

import numpy as np
import pytest
import torch

import oracle
from online_softmax_streaming_amd.workloads import random_qkv

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "f16": 2e-3, "bf16": 1e-2}
LSE_TOL = {"f32": 1e-5, "f16": 2.0 ** -11 + 1e-5, "bf16": 2.0 ** -8 + 1e-5}
DT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


@pytest.fixture(scope="module")
def lib():
    import online_softmax_streaming_amd as m
    return m


def _inputs(b, h, hkv, nq, nk, d, dtype, seed):
    q, _, _ = random_qkv(b, h, nq, nk, d, dtype, seed=seed, device="cuda")
    _, k, v = random_qkv(b, hkv, nq, nk, d, dtype, seed=seed + 1, device="cuda")
    return q, k, v


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("b,h,hkv,nq,nk,d,p", [
    (2, 4, 2, 300, 517, 128, 0.1),
    (1, 2, 2, 64, 64, 64, 0.5),
    (1, 1, 1, 5, 700, 32, 0.3),
    (2, 2, 1, 130, 33, 16, 0.9),
])
def test_parity(lib, dtype, causal, b, h, hkv, nq, nk, d, p):
    q, k, v = _inputs(b, h, hkv, nq, nk, d, dtype, seed=nq + d)
    seed, offset = 1234 + nq, 7
    out, m, l = lib.attn_fwd_dropout(q, k, v, p, seed, offset, causal=causal, want_stats=True)
    torch.cuda.synchronize()
    g = h // hkv
    want, wm, wl = oracle.attention_dropout(q.cpu().double().numpy(),
                                            np.repeat(k.cpu().double().numpy(), g, axis=1),
                                            np.repeat(v.cpu().double().numpy(), g, axis=1),
                                            causal, lib.default_scale(d), p, seed, offset)
    gain = 65536.0 / (65536.0 - oracle.threshold(p))
    err = float(np.max(np.abs(out.cpu().double().numpy() - want)))
    assert err <= TOL[dtype] * gain, err
    # Dropout leaves the row state (m, l) of the plain softmax.
    with np.errstate(divide="ignore"):
        lse = m.cpu().double().numpy() + np.log(l.cpu().double().numpy())
        wlse = wm + np.log(wl)
    fin = np.isfinite(wlse)
    assert np.array_equal(np.isfinite(lse), fin)
    assert np.max(np.abs(lse[fin] - wlse[fin]), initial=0.0) <= LSE_TOL[dtype]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("seed,offset", [(0, 0), (99, 5), (2 ** 63 + 17, 2 ** 40)])
def test_keep_decisions_are_exact(lib, dtype, causal, seed, offset):
    # Q = 0: every visible weight is exactly 1.  V = [I; 2I] over 256 keys:
    # output column c is (keep_c + 2 keep_{c+128}) * gain / l, which decodes
    # both keys' decisions.
    b, h, nq, nk, d, p = 2, 3, 300, 256, 128, 0.5
    q = torch.zeros((b, h, nq, d), dtype=DT[dtype], device="cuda")
    _, k, _ = random_qkv(b, h, nq, nk, d, dtype, seed=3, device="cuda")
    eye = torch.eye(d)
    v = torch.cat([eye, 2 * eye]).to(DT[dtype]).cuda().expand(b, h, nk, d).contiguous()
    out, _, l = lib.attn_fwd_dropout(q, k, v, p, seed, offset, causal=causal, want_stats=True)
    torch.cuda.synchronize()
    gain = 65536.0 / (65536.0 - oracle.threshold(p))
    code = np.rint(out.cpu().double().numpy() * l.cpu().double().numpy()[..., None] / gain)
    off = nk - nq
    for bi in range(b):
        for hi in range(h):
            keep = oracle.keep_mask(bi * h + hi, nq, nk, p, seed, offset)
            vis = np.ones((nq, nk), dtype=bool)
            if causal:
                vis = np.arange(nk)[None, :] <= np.arange(nq)[:, None] + off
            kv = keep & vis
            want = kv[:, :d].astype(float) + 2 * kv[:, d:].astype(float)
            assert np.array_equal(code[bi, hi], want), (bi, hi)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_p_zero_is_plain_attention(lib, dtype):
    # 32 x 4 heads: enough workgroups that the plain call takes the same
    # tiled kernel as dropout (small problems split keys over waves instead).
    q, k, v = _inputs(32, 4, 2, 300, 400, 128, dtype, seed=5)
    a, _, _ = lib.attn_fwd_dropout(q, k, v, 0.0, seed=1, causal=True)
    b = lib.attn_fwd_gqa(q, k, v, causal=True)[0]
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_same_seed_same_mask_new_offset_new_mask(lib):
    q, k, v = _inputs(1, 2, 2, 200, 200, 64, "bf16", seed=6)
    a, _, _ = lib.attn_fwd_dropout(q, k, v, 0.4, seed=10, offset=3)
    b, _, _ = lib.attn_fwd_dropout(q, k, v, 0.4, seed=10, offset=3)
    c, _, _ = lib.attn_fwd_dropout(q, k, v, 0.4, seed=10, offset=4)
    torch.cuda.synchronize()
    assert torch.equal(a, b) and not torch.equal(a, c)
