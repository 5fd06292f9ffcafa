"""GPU parity of the split softmax (softmax_rows) against the FP64 oracle.

Every case calls the HIP library through the C ABI (the Python binding
passes pointers only) and compares each output element with
oracle.softmax_rows on the same inputs, upcast exactly to FP64.

Tolerance, per element: |y - ref| <= (u + 1e-5) * ref + a, where u is the
unit roundoff of the output type (2^-24 FP32, 2^-11 FP16, 2^-8 BF16: the one
output cast) and 1e-5 covers the FP32 arithmetic before it: the exponent
formed from x - m (relative error ~|x - m| * 2^-24, |x - m| <= 60 here), the
hardware exp2 and the sum of up to 131072 terms in a tree (~(log2 N + 16) *
2^-24).  a is half the smallest subnormal spacing of the output type
(2^-25 for FP16) or 1e-37 (FP32, BF16), for outputs that round into or
below the subnormal range.
"""

import numpy as np
import pytest
import torch

import oracle

pytestmark = pytest.mark.gpu

U = {torch.float32: 2.0 ** -24, torch.float16: 2.0 ** -11, torch.bfloat16: 2.0 ** -8}
A = {torch.float32: 1e-37, torch.float16: 2.0 ** -25, torch.bfloat16: 1e-37}
DT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


def _inputs(m, n, dtype, seed, shift=0.0, ramp=0.0):
    g = torch.Generator(device="cpu").manual_seed(seed)
    x = torch.randn(m, n, generator=g, dtype=torch.float32) * 3.0
    if ramp:
        x += torch.linspace(0.0, ramp, n)  # the row maximum sits in the last chunk
    x += shift
    return x.to(dtype)


def _check(x_gpu, y_gpu, rows=None):
    dtype = x_gpu.dtype
    if rows is not None:
        idx = torch.as_tensor(rows, device=x_gpu.device)
        x_gpu, y_gpu = x_gpu[idx], y_gpu[idx]
    x = x_gpu.cpu().double().numpy()
    y = y_gpu.cpu().double().numpy()
    ref = oracle.softmax_rows(x)
    bound = (U[dtype] + 1e-5) * ref + A[dtype]
    err = np.abs(y - ref)
    assert np.all(np.isfinite(y))
    worst = float(np.max(err - bound)) if err.size else 0.0
    assert worst <= 0.0, f"max excess over the bound {worst:.3g} (max abs err {err.max():.3g})"


@pytest.fixture(scope="module")
def lib():
    import online_softmax_streaming_amd as m
    return m


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("m,n,chunk", [
    (1, 1, 256), (3, 7, 256), (2, 255, 256), (2, 256, 256), (2, 257, 256), (5, 1000, 512),
    (3, 4096, 1024), (3, 4097, 4096), (37, 333, 0), (2, 131072, 4096), (1, 131072, 256),
    (4, 32769, 1024),  # the answer-key page's A2 sizes: 33 chunks per row
])
def test_parity(lib, dtype, m, n, chunk):
    x = _inputs(m, n, DT[dtype], seed=m * 7 + n).cuda()
    y = lib.softmax_rows(x, chunk=chunk)
    torch.cuda.synchronize()
    _check(x, y)


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("shift,ramp", [(1000.0, 0.0), (-1000.0, 0.0), (0.0, 60.0)])
def test_large_logits_and_late_maximum(lib, dtype, shift, ramp):
    # Logits near +-1000 overflow or underflow exp() without the max; a ramp
    # puts every row's maximum in its last chunk, so the merge must rescale.
    x = _inputs(3, 5000, DT[dtype], seed=11, shift=shift, ramp=ramp).cuda()
    y = lib.softmax_rows(x, chunk=256)
    torch.cuda.synchronize()
    _check(x, y)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_in_place(lib, dtype):
    x = _inputs(4, 3000, DT[dtype], seed=5).cuda()
    x_copy = x.clone()
    y = lib.softmax_rows(x, chunk=512, out=x)
    torch.cuda.synchronize()
    assert y.data_ptr() == x.data_ptr()
    _check(x_copy, y)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_unaligned_rows_take_the_element_path(lib, dtype):
    # Rows of an odd length and a base 2 bytes past a 16-byte boundary.
    m, n = 3, 1001
    buf = _inputs(1, m * n + 1, DT[dtype], seed=9).reshape(-1).cuda()
    x = buf[1:].view(m, n)
    assert x.data_ptr() % 16 != 0
    y = lib.softmax_rows(x, chunk=256)
    torch.cuda.synchronize()
    _check(x, y)


def test_rows_sum_to_one(lib):
    x = _inputs(8, 20000, torch.float32, seed=3).cuda()
    y = lib.softmax_rows(x)
    torch.cuda.synchronize()
    s = y.double().sum(dim=1).cpu().numpy()
    assert np.all(np.abs(s - 1.0) <= 2e-5)


def test_empty_row_count(lib):
    x = torch.empty(0, 4096, dtype=torch.bfloat16, device="cuda")
    y = lib.softmax_rows(x)
    torch.cuda.synchronize()
    assert y.shape == (0, 4096)


def test_single_column_is_one(lib):
    x = _inputs(50, 1, torch.bfloat16, seed=2).cuda()
    y = lib.softmax_rows(x)
    torch.cuda.synchronize()
    assert torch.equal(y, torch.ones_like(y))


def test_uniform_rows_are_exact(lib):
    # exp(0) = 1 everywhere and N a power of two: 1/N is exact in every type.
    for dtype in (torch.float32, torch.float16, torch.bfloat16):
        x = torch.full((3, 4096), 2.5, dtype=dtype, device="cuda")
        y = lib.softmax_rows(x, chunk=1024)
        torch.cuda.synchronize()
        assert torch.equal(y, torch.full_like(y, 1.0 / 4096))


def test_wide_workload_sampled_rows(lib):
    # The benchmark's wide-row workload, checked on sampled rows.
    from online_softmax_streaming_amd.workloads import SOFTMAX_WORKLOADS, make_softmax_input
    w = SOFTMAX_WORKLOADS["wide_softmax_bf16"]
    x = make_softmax_input(w, seed=0, device="cuda")
    y = lib.softmax_rows(x)
    torch.cuda.synchronize()
    rows = np.random.default_rng(0).choice(w.M, 12, replace=False)
    _check(x, y, rows=rows)


def test_side_stream(lib):
    x = _inputs(6, 9000, torch.bfloat16, seed=4).cuda()
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        y = lib.softmax_rows(x, stream=s)
    s.synchronize()
    _check(x, y)


def _masked_inputs(m, n, dtype, seed):
    """Rows with runs of -inf (masked entries): a masked prefix, a run that
    straddles 16-byte vectors and chunk edges, scattered single entries, a
    fully masked row and a row masked everywhere but its last entry."""
    g = torch.Generator(device="cpu").manual_seed(seed)
    x = torch.randn(m, n, generator=g, dtype=torch.float32) * 3.0
    x[0, : min(n - 1, 300)] = float("-inf")
    x[1, 5: max(6, n // 2)] = float("-inf")
    x[2, torch.randperm(n, generator=g)[: n // 3]] = float("-inf")
    x[3, :] = float("-inf")
    x[4, :-1] = float("-inf")
    return x.to(dtype)


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("n,chunk", [(4096, 256), (1000, 256), (1001, 512), (777, 256)])
def test_masked_entries(lib, dtype, n, chunk):
    # Aligned rows (N * size a multiple of 16) take the vector path, where a
    # vector of -inf entries must give the empty state; odd N takes the
    # element path.  A fully masked row is written as zeros.
    x = _masked_inputs(6, n, DT[dtype], seed=n).cuda()
    y = lib.softmax_rows(x, chunk=chunk)
    torch.cuda.synchronize()
    _check(x, y)
    assert torch.equal(y[3], torch.zeros_like(y[3]))
    assert bool((y[x == float("-inf")] == 0).all())
