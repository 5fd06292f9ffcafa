"""GPU parity: the HIP path against the FP64 oracle, element by element.

Every call goes through the C ABI (via the ctypes binding).  Tolerances are
max abs error: 1e-5 for FP32, 2e-3 for FP16 and 1e-2 for BF16 outputs.
Small workloads are compared in full; the full-size workloads are compared on
sampled rows (first/last rows, tile edges, the ragged tail, random rows) of
sampled heads, in the same launch configuration the benchmark times.
Index work (causal visibility) is checked bit-exactly through the row state:
with Q = 0 every visible score is 0, so m = 0 and l = #visible exactly.
With $ATTN_PARITY_LOG set, every comparison appends its max abs error beside
the output-rounding floor (what an exact kernel would still show after the
one cast to the output type), so kernel error and rounding can be told apart.
"""

import json
import math
import os
import sys

import numpy as np
import pytest
import torch

import oracle
from online_softmax_streaming_amd import (attn_fwd, attn_fwd_stats, default_scale,
                                          online_merge_batch)
from online_softmax_streaming_amd.workloads import WORKLOADS, make_qkv, random_qkv

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "f16": 2e-3, "bf16": 1e-2}
# Row state (m, l) compared as log(l) + m.  On the matrix-core path l sums the
# weights after they are rounded to the input type (the same weights the P.V
# product uses), so log(l) may differ by up to that type's unit roundoff:
# 2^-8 for bf16, 2^-11 for f16; FP32 sums unrounded weights.
LSE_TOL = {"f32": 1e-5, "f16": 2.0 ** -11 + 1e-5, "bf16": 2.0 ** -8 + 1e-5}
DEV = "cuda:0"
_DT_NAME = {torch.float32: "f32", torch.float16: "f16", torch.bfloat16: "bf16"}


def _say(msg):
    print(f"[parity] {msg}", file=sys.stderr, flush=True)


_LAST_FLOOR = [0.0]


def _floor(want, dtype):
    """Output-rounding floor: max |round(o) - o| over the oracle outputs o, the
    error a kernel that computed o exactly would still show after the one
    cast to the output type."""
    if want.size == 0:
        return 0.0
    t = torch.from_numpy(np.ascontiguousarray(want))
    return float((t.to(dtype).double() - t).abs().max())


def _record(what, err, tol):
    """Append the measured error and the rounding floor of the same
    comparison to $ATTN_PARITY_LOG (JSON lines), if set."""
    path = os.environ.get("ATTN_PARITY_LOG")
    if path:
        with open(path, "a") as f:
            f.write(json.dumps({"case": what, "max_abs_err": float(err), "tol": tol,
                                "rounding_floor": _LAST_FLOOR[0]}) + "\n")


def _np(t):
    return t.detach().to("cpu", torch.float64).numpy()


def _compare_full(q, k, v, causal, scale, out, tol, m=None, l=None):
    qn, kn, vn = _np(q), _np(k), _np(v)
    want, wm, wl = oracle.attention(qn, kn, vn, causal, scale)
    got = _np(out)
    assert np.all(np.isfinite(got)), "non-finite output"
    err = np.max(np.abs(got - want)) if got.size else 0.0
    _LAST_FLOOR[0] = _floor(want, out.dtype)
    assert err <= tol, f"max abs err {err} > {tol} (rounding floor {_LAST_FLOOR[0]:.3g})"
    if m is not None:
        gm, gl = _np(m), _np(l)
        empty = wl == 0
        assert np.all(gm[empty] == -np.inf) and np.all(gl[empty] == 0)
        ok = ~empty
        # sum exp(s) = l e^m, compared as log-sum-exp.
        lse_got = gm[ok] + np.log(gl[ok])
        lse_want = wm[ok] + np.log(wl[ok])
        lse_tol = LSE_TOL[_DT_NAME[q.dtype]]
        assert np.max(np.abs(lse_got - lse_want), initial=0.0) <= lse_tol
    return err


def _sample_rows(nq, rng, extra=24):
    rows = {0, 1, 2, 31, 32, 63, 64, 127, 128, 129, nq // 2, nq - 3, nq - 2, nq - 1}
    rows |= set(int(x) for x in rng.integers(0, nq, size=extra))
    return np.array(sorted(r for r in rows if 0 <= r < nq), dtype=np.int64)


def _compare_sampled(q, k, v, causal, scale, out, tol, heads, rng):
    worst = 0.0
    _LAST_FLOOR[0] = 0.0
    for b, h in heads:
        rows = _sample_rows(q.shape[2], rng)
        want, _, _ = oracle.attention_rows(_np(q[b, h]), _np(k[b, h]), _np(v[b, h]), causal,
                                           scale, rows)
        got = _np(out[b, h, torch.as_tensor(rows, device=out.device)])
        assert np.all(np.isfinite(got))
        err = np.max(np.abs(got - want))
        _LAST_FLOOR[0] = max(_LAST_FLOOR[0], _floor(want, out.dtype))
        assert err <= tol, (f"head ({b},{h}) max abs err {err} > {tol} "
                            f"(rounding floor {_LAST_FLOOR[0]:.3g})")
        worst = max(worst, err)
    return worst


# ---------------------------------------------------------------------------
# The answer-key page's worked example on the device.
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_worked_example_six(dtype):
    _say(f"worked example dtype={dtype}")
    dt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[dtype]
    d = 16  # smallest built head size; the extra features are zero
    q = torch.zeros(1, 1, 16, d, dtype=dt)
    q[0, 0, :, 0] = 1.0
    k = torch.zeros(1, 1, 3, d, dtype=dt)
    k[0, 0, :, 0] = torch.tensor([0.0, 0.0, math.log(2.0)])
    v = torch.zeros(1, 1, 3, d, dtype=dt)
    v[0, 0, :, 0] = torch.tensor([1.0, 3.0, 10.0])
    q, k, v = q.to(DEV), k.to(DEV), v.to(DEV)
    out = attn_fwd(q, k, v, causal=False, scale=1.0)
    torch.cuda.synchronize()
    got = _np(out)[0, 0, :, 0]
    want = oracle.attention_rows(_np(q[0, 0]), _np(k[0, 0]), _np(v[0, 0]), False, 1.0)[0][:, 0]
    assert np.max(np.abs(got - want)) <= TOL[dtype]
    if dtype == "f32":
        assert np.max(np.abs(got - 6.0)) <= 1e-5
    assert np.all(_np(out)[..., 1:] == 0)


# ---------------------------------------------------------------------------
# Workloads compared in full.
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("name", ["tiny_f32", "small_causal_bf16"])
def test_small_workloads_full(name):
    w = WORKLOADS[name]
    _say(f"{name} full compare")
    q, k, v = make_qkv(w, seed=0, device=DEV)
    scale = default_scale(w.D)
    out, m, l = attn_fwd_stats(q, k, v, causal=w.causal, scale=scale)
    torch.cuda.synchronize()
    err = _compare_full(q, k, v, w.causal, scale, out, TOL[w.dtype], m, l)
    _record(name, err, TOL[w.dtype])
    _say(f"{name} max abs err {err:.3g}")


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [16, 32, 64, 128])
@pytest.mark.parametrize("nq,nk", [(259, 259), (130, 333), (333, 130), (9, 77), (64, 64)])
def test_ragged_shapes_full(dtype, causal, d, nq, nk):
    # Several query and key tiles with ragged tails, Nq != Nk in both
    # directions (causal rows with nothing visible when Nq > Nk).
    _say(f"ragged full dtype={dtype} causal={causal} D={d} Nq={nq} Nk={nk}")
    q, k, v = random_qkv(2, 3, nq, nk, d, dtype, seed=1, device=DEV, k_ramp=0.01)
    scale = default_scale(d)
    out, m, l = attn_fwd_stats(q, k, v, causal=causal, scale=scale)
    torch.cuda.synchronize()
    err = _compare_full(q, k, v, causal, scale, out, TOL[dtype], m, l)
    _record(f"ragged {dtype} causal={causal} D={d} Nq={nq} Nk={nk}", err, TOL[dtype])


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("nq,nk", [(1, 1), (1, 700), (3, 5000), (8, 4099), (5, 3)])
def test_decode_path_full(dtype, causal, nq, nk):
    # Nq <= 8 takes the split-key path: partial states + merge kernel.
    _say(f"decode full dtype={dtype} causal={causal} Nq={nq} Nk={nk}")
    q, k, v = random_qkv(2, 4, nq, nk, 128, dtype, seed=2, device=DEV, k_ramp=0.002)
    scale = default_scale(128)
    out, m, l = attn_fwd_stats(q, k, v, causal=causal, scale=scale)
    torch.cuda.synchronize()
    err = _compare_full(q, k, v, causal, scale, out, TOL[dtype], m, l)
    _record(f"decode {dtype} causal={causal} Nq={nq} Nk={nk}", err, TOL[dtype])


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("nq,nk", [(9, 8192), (17, 9000), (32, 8193), (33, 8192), (20, 8191)])
def test_decode_route_mid_rows(dtype, causal, nq, nk):
    # bf16/f16 with 9..32 rows over >= 8192 keys take the split-key path on
    # the matrix cores (rows of a head share each K/V tile read); 33 rows,
    # fewer keys and FP32 take the prefill kernels.  Same oracle either way.
    _say(f"decode route dtype={dtype} causal={causal} Nq={nq} Nk={nk}")
    q, k, v = random_qkv(2, 4, nq, nk, 128, dtype, seed=4, device=DEV, k_ramp=0.002)
    scale = default_scale(128)
    out, m, l = attn_fwd_stats(q, k, v, causal=causal, scale=scale)
    torch.cuda.synchronize()
    err = _compare_full(q, k, v, causal, scale, out, TOL[dtype], m, l)
    _record(f"decode route {dtype} causal={causal} Nq={nq} Nk={nk}", err, TOL[dtype])


# ---------------------------------------------------------------------------
# Full-size workloads, in the configuration the benchmark times.
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("name", ["headline_causal_bf16", "headline_noncausal_bf16",
                                  "ragged_causal_f16", "ragged_noncausal_f16",
                                  "long_causal_bf16"])
def test_full_size_sampled(name):
    w = WORKLOADS[name]
    _say(f"{name} sampled compare")
    q, k, v = make_qkv(w, seed=0, device=DEV)
    scale = default_scale(w.D)
    out = attn_fwd(q, k, v, causal=w.causal, scale=scale)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(out).all())
    rng = np.random.default_rng(0)
    heads = {(0, 0), (w.B - 1, w.H - 1)}
    heads |= {(int(rng.integers(w.B)), int(rng.integers(w.H))) for _ in range(2)}
    err = _compare_sampled(q, k, v, w.causal, scale, out, TOL[w.dtype], sorted(heads), rng)
    _record(name + " (sampled rows)", err, TOL[w.dtype])
    _say(f"{name} max abs err {err:.3g}")


def test_decode_workload_sampled():
    w = WORKLOADS["decode_bf16"]
    _say("decode_bf16 (B16 H32 Nq1 Nk32768 D128) sampled heads")
    q, k, v = make_qkv(w, seed=0, device=DEV)
    scale = default_scale(w.D)
    out = attn_fwd(q, k, v, causal=False, scale=scale)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(out).all())
    rng = np.random.default_rng(1)
    heads = {(0, 0), (w.B - 1, w.H - 1)}
    heads |= {(int(rng.integers(w.B)), int(rng.integers(w.H))) for _ in range(6)}
    worst = 0.0
    _LAST_FLOOR[0] = 0.0
    for b, h in sorted(heads):
        want = oracle.attention_rows(_np(q[b, h]), _np(k[b, h]), _np(v[b, h]), False, scale)[0]
        err = np.max(np.abs(_np(out[b, h]) - want))
        _LAST_FLOOR[0] = max(_LAST_FLOOR[0], _floor(want, out.dtype))
        assert err <= TOL["bf16"], f"head ({b},{h}) err {err}"
        worst = max(worst, err)
    _record("decode_bf16 (sampled heads)", worst, TOL["bf16"])
    del q, k, v, out
    torch.cuda.empty_cache()


# ---------------------------------------------------------------------------
# Degenerate cases.
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("name", ["ragged_nk1_f16", "ragged_n1_causal_f16"])
def test_single_key_is_exact(name):
    # One visible key: weight exactly 1, so out equals V's row bit for bit.
    w = WORKLOADS[name]
    _say(f"{name} bit-exact")
    q, k, v = make_qkv(w, seed=0, device=DEV)
    out, m, l = attn_fwd_stats(q, k, v, causal=w.causal)
    torch.cuda.synchronize()
    assert torch.equal(out, v[:, :, :1, :].expand_as(out))
    assert bool((l == 1).all())


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("nq", [1, 300])
@pytest.mark.parametrize("causal", [False, True])
def test_single_key_exact_all_paths(dtype, nq, causal):
    # Decode path (Nq = 1) and prefill path (Nq = 300).  Causal with Nq > Nk
    # leaves every row but the last without a visible key: those are 0.
    q, k, v = random_qkv(2, 2, nq, 1, 64, dtype, seed=3, device=DEV)
    out, m, l = attn_fwd_stats(q, k, v, causal=causal)
    torch.cuda.synchronize()
    seen = slice(nq - 1, nq) if causal else slice(0, nq)
    assert torch.equal(out[:, :, seen], v.expand_as(out[:, :, seen]))
    assert bool((l[:, :, seen] == 1).all())
    if causal:
        assert bool((out[:, :, :nq - 1] == 0).all())
        assert bool((l[:, :, :nq - 1] == 0).all())


def test_empty_batch_is_noop():
    w = WORKLOADS["ragged_b0_f16"]
    q, k, v = make_qkv(w, seed=0, device=DEV)
    out = attn_fwd(q, k, v, causal=True)
    torch.cuda.synchronize()
    assert out.shape == (0, 8, 4099, 64)


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("nq", [4, 100])
def test_no_keys_gives_zeros(dtype, nq):
    q, _, _ = random_qkv(2, 3, nq, 1, 32, dtype, seed=4, device=DEV)
    k = torch.empty((2, 3, 0, 32), dtype=q.dtype, device=DEV)
    out = torch.full_like(q, 7.0)
    out, m, l = attn_fwd_stats(q, k, k, causal=False, out=out)
    torch.cuda.synchronize()
    assert bool((out == 0).all())
    assert bool((m == -math.inf).all()) and bool((l == 0).all())


# ---------------------------------------------------------------------------
# Bit-exact causal indexing through the row state.
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("nq,nk", [(4096, 4096), (4099, 4099), (1000, 1500), (1500, 1000),
                                   (7, 1029), (257, 64), (1, 5)])
def test_causal_visible_counts_exact(dtype, nq, nk):
    _say(f"visible counts dtype={dtype} Nq={nq} Nk={nk}")
    _, k, v = random_qkv(1, 2, nq, nk, 64, dtype, seed=5, device=DEV)
    q = torch.zeros((1, 2, nq, 64), dtype=k.dtype, device=DEV)
    out, m, l = attn_fwd_stats(q, k, v, causal=True)
    torch.cuda.synchronize()
    want = oracle.visible_mask(nq, nk, True).sum(axis=1).astype(np.float64)
    gl = _np(l)
    gm = _np(m)
    for h in range(2):
        assert np.array_equal(gl[0, h], want), "visible-key count differs"
        assert np.all(gm[0, h][want > 0] == 0) and np.all(gm[0, h][want == 0] == -np.inf)


# ---------------------------------------------------------------------------
# Streams, repeatability and the device merge.
# ---------------------------------------------------------------------------

def test_side_stream_and_repeatability():
    w = WORKLOADS["small_causal_bf16"]
    q, k, v = make_qkv(w, seed=7, device=DEV)
    ref = attn_fwd(q, k, v, causal=True)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        out2 = attn_fwd(q, k, v, causal=True, stream=s)
    s.synchronize()
    torch.cuda.synchronize()
    assert torch.equal(ref, out2)


def test_online_merge_batch_matches_oracle():
    rng = np.random.default_rng(8)
    n = 10007
    m1 = rng.normal(size=n) * 10
    m2 = rng.normal(size=n) * 10
    l1 = rng.uniform(0.01, 100, size=n)
    l2 = rng.uniform(0.01, 100, size=n)
    e1 = rng.uniform(size=n) < 0.1
    e2 = rng.uniform(size=n) < 0.1
    m1[e1], l1[e1] = -np.inf, 0.0
    m2[e2], l2[e2] = -np.inf, 0.0
    m1[:3] = [2.0, -np.inf, 7.0]
    l1[:3] = [2.0, 0.0, 1.0]
    m2[:3] = [4.0, -np.inf, -np.inf]
    l2[:3] = [1.0, 0.0, 0.0]
    t = [torch.tensor(x, dtype=torch.float32, device=DEV) for x in (m1, l1, m2, l2)]
    gm, gl = online_merge_batch(*t)
    torch.cuda.synchronize()
    wm, wl = oracle.online_merge(*(x.cpu().double().numpy() for x in t))
    gm, gl = gm.cpu().double().numpy(), gl.cpu().double().numpy()
    assert np.array_equal(gm, wm)
    assert not np.isnan(gl).any()
    assert np.max(np.abs(gl - wl) / np.maximum(wl, 1e-30)) <= 1e-6
    assert gm[1] == -np.inf and gl[1] == 0.0
    assert abs(gl[0] - (1 + 2 * math.exp(-2))) <= 1e-6


# ---------------------------------------------------------------------------
# Grid-size variants of the tiled kernel.
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("nq,nk,d", [(259, 259, 128), (130, 333, 64), (333, 130, 64),
                                     (64, 64, 32), (700, 700, 16), (40, 2000, 64),
                                     (100, 1000, 128), (64, 4099, 128)])
def test_small_grid_split_and_wide_grid(dtype, causal, nq, nk, d):
    # A problem with few workgroups splits the keys of each 32-row block over
    # the waves of a workgroup and merges their states; a large one streams
    # them in one wave.  Both are checked against the oracle: the small
    # problem in full, the same heads repeated 96 times (at least 192
    # eight-wave workgroups, which take eight-wave workgroups of the tiled
    # kernel) on three repeats.  At D = 128 the split waves stage each next tile in
    # registers: 4099 keys give a wave 16 or 17 tiles, the last one ragged.
    _say(f"grid variants dtype={dtype} causal={causal} Nq={nq} Nk={nk} D={d}")
    q, k, v = random_qkv(1, 2, nq, nk, d, dtype, seed=nq + 7 * nk + d, device=DEV, k_ramp=0.01)
    scale = default_scale(d)
    small, sm, sl = attn_fwd_stats(q, k, v, causal=causal, scale=scale)
    wide, wm, wl = attn_fwd_stats(q.repeat(96, 1, 1, 1), k.repeat(96, 1, 1, 1),
                                  v.repeat(96, 1, 1, 1), causal=causal, scale=scale)
    again = attn_fwd(q, k, v, causal=causal, scale=scale)
    torch.cuda.synchronize()
    assert torch.equal(again, small), "the split path is not deterministic"
    err = _compare_full(q, k, v, causal, scale, small, TOL[dtype], sm, sl)
    _record(f"small grid {dtype} causal={causal} D={d} Nq={nq} Nk={nk}", err, TOL[dtype])
    for rep in (0, 47, 95):
        _compare_full(q, k, v, causal, scale, wide[rep:rep + 1], TOL[dtype], wm[rep:rep + 1],
                      wl[rep:rep + 1])


@pytest.mark.parametrize("b,h,n,d,causal,dtype", [
    # 64 eight-wave workgroups, the most the key-split path takes at D <= 64.
    (1, 8, 2048, 64, False, "bf16"), (2, 4, 4096, 64, True, "bf16"),
    (2, 8, 2048, 32, True, "bf16"), (2, 4, 2048, 16, False, "f16"),
    # 65 to 128 eight-wave workgroups: four-wave workgroups of 128 rows.
    (1, 8, 8192, 64, True, "bf16"), (1, 8, 4096, 128, False, "bf16"),
    (1, 12, 2048, 64, False, "f16"), (2, 4, 4100, 128, True, "bf16")])
def test_grid_size_paths(b, h, n, d, causal, dtype):
    # The paths the launch takes by grid size, at their boundaries: heads 0
    # and the last one compared in full.
    _say(f"grid-size path B={b} H={h} N={n} D={d} causal={causal} {dtype}")
    q, k, v = random_qkv(b, h, n, n, d, dtype, seed=n + d, device=DEV, k_ramp=0.002)
    scale = default_scale(d)
    out, m, l = attn_fwd_stats(q, k, v, causal=causal, scale=scale)
    torch.cuda.synchronize()
    err = 0.0
    for bi, hi in [(0, 0), (b - 1, h - 1)]:
        sl = (slice(bi, bi + 1), slice(hi, hi + 1))
        err = max(err, _compare_full(q[sl], k[sl], v[sl], causal, scale, out[sl], TOL[dtype],
                                     m[sl], l[sl]))
    _record(f"grid-size path B={b} H={h} N={n} D={d} causal={causal} {dtype}", err, TOL[dtype])


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("nq,nk", [(700, 700), (700, 1000), (1000, 333)])
def test_sixteen_wave_noncausal_d64(dtype, nq, nk):
    # Noncausal D = 64 with 100 heads of 700-1000 rows: eight-wave
    # workgroups would number more than the 256 CUs, sixteen-wave ones (512
    # rows) fit once, so the launch takes the sixteen-wave kernel.  Three
    # repeats of the two distinct heads are compared in full.
    _say(f"sixteen-wave D=64 dtype={dtype} Nq={nq} Nk={nk}")
    q, k, v = random_qkv(1, 2, nq, nk, 64, dtype, seed=nq + nk, device=DEV, k_ramp=0.01)
    scale = default_scale(64)
    wide, wm, wl = attn_fwd_stats(q.repeat(50, 1, 1, 1), k.repeat(50, 1, 1, 1),
                                  v.repeat(50, 1, 1, 1), causal=False, scale=scale)
    torch.cuda.synchronize()
    err = 0.0
    for rep in (0, 23, 49):
        err = max(err, _compare_full(q, k, v, False, scale, wide[rep:rep + 1], TOL[dtype],
                                     wm[rep:rep + 1], wl[rep:rep + 1]))
    _record(f"sixteen-wave {dtype} D=64 Nq={nq} Nk={nk}", err, TOL[dtype])


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("nq,nk,d", [(259, 259, 128), (130, 333, 64), (333, 130, 32),
                                     (100, 100, 16)])
def test_fp32_small_grid_split_and_default_split(causal, nq, nk, d):
    # FP32 problems with few workgroups split each row over D/4 threads,
    # large ones over 1 or 2.  The summation order differs, so both are
    # checked against the oracle: the small problem in full, the same heads
    # repeated 256 times (at least 512 default workgroups) on three of the
    # repeats.
    _say(f"fp32 grid variants causal={causal} Nq={nq} Nk={nk} D={d}")
    q, k, v = random_qkv(1, 2, nq, nk, d, "f32", seed=nq + 3 * nk + d, device=DEV, k_ramp=0.01)
    scale = default_scale(d)
    small, sm, sl = attn_fwd_stats(q, k, v, causal=causal, scale=scale)
    wide, wm, wl = attn_fwd_stats(q.repeat(256, 1, 1, 1), k.repeat(256, 1, 1, 1),
                                  v.repeat(256, 1, 1, 1), causal=causal, scale=scale)
    torch.cuda.synchronize()
    err = _compare_full(q, k, v, causal, scale, small, TOL["f32"], sm, sl)
    _record(f"fp32 small grid causal={causal} D={d} Nq={nq} Nk={nk}", err, TOL["f32"])
    for rep in (0, 137, 255):
        _compare_full(q, k, v, causal, scale, wide[rep:rep + 1], TOL["f32"], wm[rep:rep + 1],
                      wl[rep:rep + 1])


@pytest.mark.parametrize("b,h,nq,nk,d,causal,dtype", [
    # Few 256-row query tiles over many keys: the keys of each tile are split
    # over workgroups and the partial states combined (4 to 64 splits; ragged
    # query tiles, a ragged last split and key tile).
    (1, 4, 256, 8192, 128, True, "bf16"), (1, 1, 512, 65536, 128, True, "bf16"),
    (1, 1, 1000, 20000, 64, False, "f16"), (2, 1, 300, 12000, 128, False, "bf16"),
    (1, 2, 256, 16384, 32, True, "bf16"), (1, 1, 512, 32768, 16, False, "f16"),
    # Causal with Nq = Nk: splits past the diagonal see no key of their rows.
    (1, 1, 8192, 8192, 128, True, "bf16"),
    # More rows than keys, causal: the first Nq - Nk rows see no key at all.
    (1, 1, 8200, 8192, 128, True, "bf16")])
def test_split_kv_route(b, h, nq, nk, d, causal, dtype):
    # Every head compared in full, row states included, and the result
    # repeatable bit for bit.
    _say(f"split-kv B={b} H={h} Nq={nq} Nk={nk} D={d} causal={causal} {dtype}")
    q, k, v = random_qkv(b, h, nq, nk, d, dtype, seed=nq + nk + d, device=DEV, k_ramp=0.002)
    scale = default_scale(d)
    out, m, l = attn_fwd_stats(q, k, v, causal=causal, scale=scale)
    again = attn_fwd(q, k, v, causal=causal, scale=scale)
    torch.cuda.synchronize()
    assert torch.equal(again, out), "the split-kv path is not deterministic"
    err = _compare_full(q, k, v, causal, scale, out, TOL[dtype], m, l)
    _record(f"split-kv B={b} H={h} Nq={nq} Nk={nk} D={d} causal={causal} {dtype}", err,
            TOL[dtype])


@pytest.mark.parametrize("b,h,nq,nk,d,causal", [
    (1, 8, 512, 8192, 64, True), (1, 2, 4096, 4096, 128, True),
    (1, 4, 1000, 9000, 32, False), (1, 2, 700, 33000, 16, True)])
def test_split_kv_route_f32(b, h, nq, nk, d, causal):
    # FP32 problems too small for the default kernel to fill the GPU, over
    # long keys: each query tile's keys split over workgroups of the default
    # kernel (8 to 64 splits; ragged tiles) and combined.  Unramped keys keep
    # the logits where FP32 scores carry the 1e-5 bound.
    _say(f"split-kv f32 B={b} H={h} Nq={nq} Nk={nk} D={d} causal={causal}")
    q, k, v = random_qkv(b, h, nq, nk, d, "f32", seed=nq + nk + d, device=DEV)
    scale = default_scale(d)
    out, m, l = attn_fwd_stats(q, k, v, causal=causal, scale=scale)
    again = attn_fwd(q, k, v, causal=causal, scale=scale)
    torch.cuda.synchronize()
    assert torch.equal(again, out), "the split-kv path is not deterministic"
    err = _compare_full(q, k, v, causal, scale, out, TOL["f32"], m, l)
    _record(f"split-kv f32 B={b} H={h} Nq={nq} Nk={nk} D={d} causal={causal}", err, TOL["f32"])
