"""Properties of the GPU result that hold whatever the inputs' values.

These complement the element-wise parity against the FP64 oracle with
checks whose expected values come from the mathematics alone:

* uniform weights: with Q = 0 every visible score is 0, every weight is
  exactly 1, and each output row is the mean of the value rows the row may
  see.  With V[j, :] = j that mean is (first + last visible key) / 2, which
  pins which keys each row sees (causal rule with the diagonal included,
  bottom-right alignment when Nq != Nk) in every dtype and on both paths;
* shift invariance: adding one constant to every score of a row leaves the
  softmax unchanged.  The shift rides on a padded feature (Q[..., D-1] = 1,
  K[..., D-1] = c), up to scores ~125 above the rest, where exp without the
  max subtraction would overflow FP32;
* permutation invariance (noncausal: permuting K and V rows together changes
  only the summation order) and convexity (every output lies within the
  range of the value column it averages).
"""

import numpy as np
import pytest
import torch

import oracle
from online_softmax_streaming_amd import attn_fwd, default_scale
from online_softmax_streaming_amd.workloads import random_qkv

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "f16": 2e-3, "bf16": 1e-2}
DT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


def _ramp_values(b, h, nk, d, dtype):
    j = torch.arange(nk, dtype=torch.float32, device="cuda")
    return j[None, None, :, None].expand(b, h, nk, d).to(DT[dtype]).contiguous()


@pytest.mark.parametrize("dtype,nq,nk,causal", [
    ("f32", 300, 300, True), ("f32", 1029, 1029, True), ("f32", 130, 517, True),
    ("f32", 77, 200, False),
    ("bf16", 256, 256, True), ("bf16", 100, 257, True), ("bf16", 64, 200, False),
    ("f16", 1029, 1029, True), ("f16", 300, 700, True), ("f16", 5, 900, True),
    ("bf16", 3, 200, True), ("f32", 8, 1000, False),
])
def test_uniform_weights_give_mean_of_visible_values(dtype, nq, nk, causal):
    # Every value used here (keys 0..nk-1, half-integers up to (nk-1)/2) is
    # exact in the dtype, and the FP32 sums of at most 1029 integers are
    # exact; the only rounding is the final division, at most 1 ulp of FP32.
    d = 64
    q = torch.zeros((2, 2, nq, d), dtype=DT[dtype], device="cuda")
    k = random_qkv(2, 2, nq, nk, d, dtype, seed=nq + nk, device="cuda")[1]
    v = _ramp_values(2, 2, nk, d, dtype)
    out = attn_fwd(q, k, v, causal=causal)
    torch.cuda.synchronize()
    got = out.double().cpu().numpy()
    off = nk - nq
    last = np.arange(nq) + off if causal else np.full(nq, nk - 1)
    want = np.where(last >= 0, np.maximum(last, 0) / 2.0, 0.0)
    rel = np.abs(got - want[None, None, :, None]) / np.maximum(want[None, None, :, None], 1.0)
    # FP32: a * fl(1/l) is within two roundings of the mean; the narrower
    # types then round back to the mean itself, which they represent.
    bound = 2.0 ** -22 if dtype == "f32" else 0.0
    assert float(rel.max()) <= bound, f"worst relative deviation {rel.max():.3g}"


def _score_rounding_bound(qd, kd, vd, scale):
    """Extra output error that FP32 score arithmetic allows once scores are
    large: a dot product of D terms accumulated in FP32 is off by at most
    about (D + 2) * 2^-24 * max|score| (any summation order), which moves
    every weight by that relative amount and the output by twice that times
    max|V|."""
    s_max = float(np.max(np.abs(np.einsum("bhqd,bhkd->bhqk", qd, kd)))) * scale
    return (qd.shape[-1] + 2) * 2.0 ** -24 * s_max * 2 * float(np.max(np.abs(vd)))


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("causal", [False, True])
def test_shift_invariance_with_large_scores(dtype, causal):
    b, h, nq, nk, d = 1, 2, 200, 333, 64
    q, k, v = random_qkv(b, h, nq, nk, d, dtype, seed=21, device="cuda")
    q[..., d - 1] = 1.0
    scale = default_scale(d)
    outs = []
    for shift in (0.0, 96.0, 1000.0):  # scores rise by shift / 8, up to 125 (exp overflows at 88.7)
        k[..., d - 1] = shift
        out = attn_fwd(q, k, v, causal=causal, scale=scale)
        torch.cuda.synchronize()
        got = out.double().cpu().numpy()
        assert np.all(np.isfinite(got)), f"non-finite output at shift {shift}"
        qd, kd, vd = (t.double().cpu().numpy() for t in (q, k, v))
        want, _, _ = oracle.attention(qd, kd, vd, causal, scale)
        tol = TOL[dtype] + _score_rounding_bound(qd, kd, vd, scale)
        err = float(np.max(np.abs(got - want)))
        assert err <= tol, f"shift {shift}: max abs err {err:.3g} > {tol:.3g}"
        outs.append((got, tol))
    for got, tol in outs[1:]:
        assert float(np.max(np.abs(got - outs[0][0]))) <= tol + outs[0][1]


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_permutation_invariance_and_convexity(dtype):
    b, h, nq, nk, d = 1, 3, 150, 413, 128
    q, k, v = random_qkv(b, h, nq, nk, d, dtype, seed=22, device="cuda")
    out = attn_fwd(q, k, v, causal=False)
    perm = torch.from_numpy(np.random.default_rng(23).permutation(nk)).to("cuda")
    out_p = attn_fwd(q, k[:, :, perm].contiguous(), v[:, :, perm].contiguous(), causal=False)
    torch.cuda.synchronize()
    got, got_p = out.double().cpu().numpy(), out_p.double().cpu().numpy()
    assert float(np.max(np.abs(got - got_p))) <= 2 * TOL[dtype]
    vd = v.double().cpu().numpy()
    lo = vd.min(axis=2, keepdims=True)
    hi = vd.max(axis=2, keepdims=True)
    # FP32 accumulation over nk weighted terms (at most nk * 2^-24 of max|V|
    # relative to the weight sum), then the output cast (one ulp allowed).
    ulp = {"f32": 2.0 ** -23, "f16": 2.0 ** -10, "bf16": 2.0 ** -7}[dtype]
    slack = (nk * 2.0 ** -24 + ulp) * np.maximum(np.abs(lo), np.abs(hi))
    assert np.all(got >= lo - slack) and np.all(got <= hi + slack)
