"""Host-side checks of the C ABI (no GPU needed).

The library must load, export every symbol include/attn.h declares, reject
bad arguments before touching any device, and compute the host A1 merge to
the oracle's values.  None of these calls launches a kernel.
"""

import math
import os
import re

import numpy as np
import pytest

from oracle import online_merge as oracle_merge

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn.h")


@pytest.fixture(scope="module")
def attn():
    from online_softmax_streaming_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        from online_softmax_streaming_amd import build
        build.build()
    import online_softmax_streaming_amd as m
    return m


def _declared_symbols():
    text = open(HEADER).read()
    return re.findall(r"ATTN_API\s+[\w\s\*]+?\b(\w+)\s*\(", text)


def test_header_declares_the_boundary():
    names = set(_declared_symbols())
    assert {"attn_fwd", "attn_fwd_stats", "online_merge", "online_merge_batch",
            "attn_strerror", "attn_last_error"} <= names


def test_library_exports_every_declared_symbol(attn):
    import subprocess
    from online_softmax_streaming_amd import _lib
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    for name in _declared_symbols():
        assert name in exported, name
        assert hasattr(_lib.lib(), name)
    # Only the C ABI is exported.
    assert exported == set(_declared_symbols())


def test_library_is_a_gfx950_build(attn):
    from online_softmax_streaming_amd import _lib
    blob = open(_lib.LIB_PATH, "rb").read()
    assert b"gfx950" in blob


def test_strerror(attn):
    assert attn.attn_strerror(0) == "success"
    assert attn.attn_strerror(1) == "invalid argument"
    assert attn.attn_strerror(2) == "unsupported configuration"
    assert attn.attn_strerror(3) == "HIP runtime error"
    assert attn.attn_strerror(99) == "unknown status code"


def test_host_merge_worked_example(attn):
    # Answer-key page, worked answer A1.
    m, l = attn.online_merge(2.0, 2.0, 4.0, 1.0)
    assert m == 4.0
    assert abs(l - (1 + 2 * math.exp(-2))) <= 4e-16


def test_host_merge_empty_cases(attn):
    inf = float("inf")
    assert attn.online_merge(-inf, 0.0, -inf, 0.0) == (-inf, 0.0)
    assert attn.online_merge(1.5, 3.0, -inf, 0.0) == (1.5, 3.0)
    assert attn.online_merge(-inf, 0.0, -7.0, 0.25) == (-7.0, 0.25)


def test_host_merge_matches_oracle(attn):
    rng = np.random.default_rng(0)
    for _ in range(500):
        m1, m2 = rng.normal(size=2) * 20
        l1, l2 = rng.uniform(0, 100, size=2)
        if rng.uniform() < 0.1:
            m1, l1 = -math.inf, 0.0
        got = attn.online_merge(m1, l1, m2, l2)
        want = oracle_merge(m1, l1, m2, l2)
        assert got[0] == want[0]
        assert abs(got[1] - want[1]) <= 1e-15 * max(1.0, want[1])


@pytest.mark.parametrize("args", [
    (float("nan"), 1.0, 0.0, 1.0),
    (float("inf"), 1.0, 0.0, 1.0),
    (0.0, -1.0, 0.0, 1.0),
    (0.0, 1.0, 0.0, float("nan")),
    (0.0, float("inf"), 0.0, 1.0),
])
def test_host_merge_rejects_bad_states(attn, args):
    with pytest.raises(attn.AttnError) as e:
        attn.online_merge(*args)
    assert e.value.code == attn.ATTN_E_INVALID


def _raw(attn, **kw):
    args = dict(q_ptr=0x1000, k_ptr=0x2000000, v_ptr=0x4000000, out_ptr=0x8000000, b=1, h=1,
                nq=16, nk=16, d=64, causal=0, scale=0.125, dtype=attn.ATTN_BF16)
    args.update(kw)
    return attn.attn_fwd_raw(**args)


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=7), 1),
    (dict(causal=2), 1),
    (dict(b=-1), 1),
    (dict(nk=-3), 1),
    (dict(d=0), 1),
    (dict(scale=0.0), 1),
    (dict(scale=-0.5), 1),
    (dict(scale=float("nan")), 1),
    (dict(scale=float("inf")), 1),
    (dict(d=48), 2),
    (dict(d=256), 2),
    (dict(q_ptr=0), 1),
    (dict(out_ptr=0), 1),
    (dict(k_ptr=0), 1),
    (dict(q_ptr=0x1008), 1),            # misaligned
    (dict(out_ptr=0x1000 + 1024), 1),   # out overlaps Q
    (dict(nq=1 << 31), 1),
    (dict(nk=(1 << 31) // 64), 1),      # Nk*D reaches 2^31
    (dict(b=1 << 16, h=1 << 16), 1),    # B*H reaches 2^32
])
def test_attn_fwd_rejects_bad_arguments(attn, kw, code):
    assert _raw(attn, **kw) == code


@pytest.mark.parametrize("kw", [dict(b=0), dict(h=0), dict(nq=0),
                                dict(b=0, q_ptr=0, k_ptr=0, v_ptr=0, out_ptr=0)])
def test_attn_fwd_empty_is_a_noop(attn, kw):
    # B, H or Nq == 0 returns before any device work, whatever the pointers.
    assert _raw(attn, **kw) == 0


def test_last_error_text(attn):
    from online_softmax_streaming_amd import _lib
    assert _raw(attn, d=48) == 2
    assert "D=48" in _lib.lib().attn_last_error().decode()
    assert _raw(attn, scale=-1.0) == 1
    assert "scale" in _lib.lib().attn_last_error().decode()


def test_merge_batch_rejects_bad_sizes(attn):
    from online_softmax_streaming_amd import _lib
    L = _lib.lib()
    import ctypes
    p = ctypes.c_void_p(0x1000)
    assert L.online_merge_batch(p, p, p, p, p, p, -1, None) == 1
    assert L.online_merge_batch(p, p, p, p, p, p, 0, None) == 0
    assert L.online_merge_batch(None, p, p, p, p, p, 4, None) == 1
    assert L.online_merge_batch(ctypes.c_void_p(0x1001), p, p, p, p, p, 4, None) == 1


# --------------------------------------------------------------------------
# Split softmax: host-side sizing and argument checks (no kernel launched).

def test_softmax_scratch_worked_example(attn):
    # Answer-key page, worked answer A2: M=4, N=32769, C=1024 -> T=33 chunks,
    # 8*4*(33+1) = 1088 bytes of scratch.
    import json
    g = json.load(open(os.path.join(ROOT, "tests", "golden", "worked_examples.json")))["a2_scratch"]
    assert attn.softmax_rows_scratch_bytes(g["M"], g["N"], g["chunk"]) == g["expected_scratch_bytes"]


@pytest.mark.parametrize("m,n,c", [(1, 1, 256), (3, 256, 256), (3, 257, 256), (2, 131072, 4096),
                                   (0, 5, 1024), (7, 100000, 512)])
def test_softmax_scratch_matches_oracle_formula(attn, m, n, c):
    from oracle import scratch_bytes
    assert attn.softmax_rows_scratch_bytes(m, n, c) == scratch_bytes(m, n, c)


def test_softmax_scratch_auto_chunk_is_a_listed_size(attn):
    from oracle import scratch_bytes
    for m, n in ((1, 131072), (4096, 4096), (4, 32769), (100000, 300)):
        got = attn.softmax_rows_scratch_bytes(m, n, 0)
        assert got in {scratch_bytes(m, n, c) for c in (256, 512, 1024, 2048, 4096)}


@pytest.mark.parametrize("m,n,c", [(-1, 5, 256), (2, 0, 256), (2, 5, 100), (2, 5, 8192)])
def test_softmax_scratch_rejects_bad_sizes(attn, m, n, c):
    assert attn.softmax_rows_scratch_bytes(m, n, c) == -1


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=7), 1),
    (dict(M=-1), 1),
    (dict(N=0), 1),
    (dict(chunk=300), 1),
    (dict(x=0), 1),
    (dict(y=0), 1),
    (dict(x=17), 1),              # not aligned to the element size
    (dict(y=4104), 1),            # overlaps x without being x
    (dict(M=1 << 31, N=4096, chunk=256, y=4096), 2),  # in place; too many chunks for one grid
])
def test_softmax_rows_rejects_bad_arguments(attn, kw, code):
    from online_softmax_streaming_amd import _lib
    args = dict(x=4096, y=1 << 30, M=4, N=1024, chunk=256, dtype=2, stream=None)
    args.update(kw)
    rc = _lib.lib().softmax_rows(args["x"], args["y"], args["M"], args["N"], args["chunk"],
                                 args["dtype"], args["stream"])
    assert rc == code, _lib.lib().attn_last_error()


def test_softmax_rows_empty_is_a_noop(attn):
    from online_softmax_streaming_amd import _lib
    assert _lib.lib().softmax_rows(None, None, 0, 1024, 0, 2, None) == 0


@pytest.mark.parametrize("hkv", [0, -1, 3, 16])
def test_attn_fwd_gqa_rejects_bad_group(attn, hkv):
    from online_softmax_streaming_amd import _lib
    rc = _lib.lib().attn_fwd_gqa(4096, 8192, 12288, 1 << 30, 1, 8, hkv, 64, 64, 64, 0, 0.125, 2,
                                 None, None, None)
    assert rc == 1, _lib.lib().attn_last_error()
    assert b"Hkv" in _lib.lib().attn_last_error()


def _bwd(attn, **kw):
    from online_softmax_streaming_amd import _lib
    g = 1 << 24  # fake, disjoint device addresses: every case fails before any device call
    a = dict(q=1 * g, k=2 * g, v=3 * g, o=4 * g, do=5 * g, m=6 * g, l=7 * g, dq=8 * g, dk=9 * g,
             dv=10 * g, b=1, h=2, hkv=2, nq=64, nk=64, d=64, causal=0, scale=0.125, dtype=2)
    a.update(kw)
    return _lib.lib().attn_bwd(a["q"], a["k"], a["v"], a["o"], a["do"], a["m"], a["l"], a["dq"],
                               a["dk"], a["dv"], a["b"], a["h"], a["hkv"], a["nq"], a["nk"],
                               a["d"], a["causal"], a["scale"], a["dtype"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=0, d=48), 2),                 # FP32: D not built
    (dict(dtype=0, dq=(1 << 24) + 24576), 1),  # FP32 (4-byte elements): dQ overlaps Q
    (dict(dtype=7), 1),
    (dict(causal=2), 1),
    (dict(hkv=3), 1),
    (dict(hkv=0), 1),
    (dict(d=48), 2),
    (dict(scale=0.0), 1),
    (dict(scale=float("nan")), 1),
    (dict(nq=-1), 1),
    (dict(q=0), 1),
    (dict(o=0), 1),
    (dict(do=0), 1),
    (dict(m=0), 1),
    (dict(dq=0), 1),
    (dict(dk=0), 1),
    (dict(v=0), 1),
    (dict(q=(1 << 24) + 8), 1),               # misaligned
    (dict(m=6 * (1 << 24) + 2), 1),           # misaligned row state
    (dict(dq=(1 << 24) + 1024), 1),           # dQ overlaps Q
    (dict(dk=10 * (1 << 24)), 1),             # dK is dV
    (dict(dv=6 * (1 << 24)), 1),              # dV overlaps m
    (dict(nq=1, b=1 << 16, h=1 << 8, hkv=1 << 8, nk=1 << 8), 1),  # B*Hkv*Nk reaches 2^32
    (dict(nk=(1 << 31) // 64), 1),            # Nk*D reaches 2^31
])
def test_attn_bwd_rejects_bad_arguments(attn, kw, code):
    from online_softmax_streaming_amd import _lib
    assert _bwd(attn, **kw) == code, _lib.lib().attn_last_error()


@pytest.mark.parametrize("kw", [dict(b=0), dict(h=0), dict(nq=0, nk=0),
                                dict(b=0, q=0, k=0, v=0, o=0, do=0, m=0, l=0, dq=0, dk=0, dv=0)])
def test_attn_bwd_empty_is_a_noop(attn, kw):
    assert _bwd(attn, **kw) == 0


def _paged(attn, **kw):
    from online_softmax_streaming_amd import _lib
    g = 1 << 24
    a = dict(q=1 * g, kc=2 * g, vc=4 * g, table=6 * g, lens=7 * g, out=8 * g, b=2, h=4, hkv=2,
             nq=1, d=64, num_pages=16, page_size=16, max_pages=8, causal=1, window=0,
             scale=0.125, dtype=2, m=None, l=None)
    a.update(kw)
    return _lib.lib().attn_decode_paged(a["q"], a["kc"], a["vc"], a["table"], a["lens"], a["out"],
                                        a["b"], a["h"], a["hkv"], a["nq"], a["d"],
                                        a["num_pages"], a["page_size"], a["max_pages"],
                                        a["causal"], a["window"], a["scale"], a["dtype"],
                                        a["m"], a["l"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=7), 1),
    (dict(causal=2), 1),
    (dict(hkv=3), 1),
    (dict(d=48), 2),
    (dict(scale=-1.0), 1),
    (dict(window=-1), 1),
    (dict(window=4, causal=0), 1),          # a window needs causal attention
    (dict(page_size=12), 1),                # not a power of two
    (dict(page_size=0), 1),
    (dict(num_pages=0), 1),
    (dict(max_pages=0), 1),
    (dict(max_pages=1 << 27, page_size=16), 1),  # max_pages * page_size reaches 2^31
    (dict(q=0), 1),
    (dict(table=0), 1),
    (dict(lens=0), 1),
    (dict(kc=2 * (1 << 24) + 8), 1),        # misaligned cache
    (dict(table=6 * (1 << 24) + 2), 1),     # misaligned table
    (dict(out=2 * (1 << 24)), 1),           # out overlaps K_cache
    (dict(out=6 * (1 << 24)), 1),           # out overlaps the table
])
def test_attn_decode_paged_rejects_bad_arguments(attn, kw, code):
    from online_softmax_streaming_amd import _lib
    assert _paged(attn, **kw) == code, _lib.lib().attn_last_error()


@pytest.mark.parametrize("kw", [dict(b=0), dict(h=0), dict(nq=0),
                                dict(b=0, q=0, kc=0, vc=0, table=0, lens=0, out=0)])
def test_attn_decode_paged_empty_is_a_noop(attn, kw):
    assert _paged(attn, **kw) == 0


def _varlen(attn, **kw):
    from online_softmax_streaming_amd import _lib
    g = 1 << 24
    a = dict(q=1 * g, k=2 * g, v=3 * g, out=4 * g, cq=5 * g, ck=6 * g, b=3, h=4, hkv=2,
             tq=300, tk=500, mq=200, d=64, causal=1, scale=0.125, dtype=2, m=None, l=None)
    a.update(kw)
    return _lib.lib().attn_fwd_varlen(a["q"], a["k"], a["v"], a["out"], a["cq"], a["ck"], a["b"],
                                      a["h"], a["hkv"], a["tq"], a["tk"], a["mq"], a["d"],
                                      a["causal"], a["scale"], a["dtype"], a["m"], a["l"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=7), 1),
    (dict(causal=2), 1),
    (dict(hkv=3), 1),
    (dict(d=48), 2),
    (dict(scale=0.0), 1),
    (dict(tq=-1), 1),
    (dict(mq=301), 1),                    # longer than total_q
    (dict(q=0), 1),
    (dict(cq=0), 1),
    (dict(ck=0), 1),
    (dict(k=0), 1),
    (dict(q=(1 << 24) + 8), 1),           # misaligned
    (dict(cq=5 * (1 << 24) + 2), 1),      # misaligned offsets
    (dict(out=(1 << 24) + 64), 1),        # out overlaps Q
    (dict(tk=1 << 24, hkv=2, d=64), 2),   # packed K above 4 GiB
    (dict(tq=1 << 31), 1),
])
def test_attn_fwd_varlen_rejects_bad_arguments(attn, kw, code):
    from online_softmax_streaming_amd import _lib
    assert _varlen(attn, **kw) == code, _lib.lib().attn_last_error()


@pytest.mark.parametrize("kw", [dict(b=0), dict(h=0), dict(tq=0, mq=0),
                                dict(b=0, q=0, k=0, v=0, out=0, cq=0, ck=0)])
def test_attn_fwd_varlen_empty_is_a_noop(attn, kw):
    assert _varlen(attn, **kw) == 0


def _masked(attn, **kw):
    from online_softmax_streaming_amd import _lib
    g = 1 << 24
    a = dict(q=1 * g, k=2 * g, v=3 * g, out=4 * g, mask=5 * g, sb=0, sh=0, b=2, h=4, hkv=2,
             nq=64, nk=64, d=64, causal=1, window=0, scale=0.125, dtype=2)
    a.update(kw)
    return _lib.lib().attn_fwd_masked(a["q"], a["k"], a["v"], a["out"], a["mask"], a["sb"], a["sh"],
                                      a["b"], a["h"], a["hkv"], a["nq"], a["nk"], a["d"],
                                      a["causal"], a["window"], a["scale"], a["dtype"], None, None,
                                      None)


@pytest.mark.parametrize("kw,code", [
    (dict(window=-1), 1),
    (dict(window=8, causal=0), 1),
    (dict(sb=-1), 1),
    (dict(mask=5 * (1 << 24) + 2), 1),          # misaligned mask
    (dict(out=5 * (1 << 24)), 1),               # out overlaps the mask
    (dict(d=48), 2),
    (dict(hkv=3), 1),
])
def test_attn_fwd_masked_rejects_bad_arguments(attn, kw, code):
    from online_softmax_streaming_amd import _lib
    assert _masked(attn, **kw) == code, _lib.lib().attn_last_error()


@pytest.mark.parametrize("p", [-0.1, 1.0, float("nan"), 0.999995])
def test_attn_fwd_dropout_rejects_bad_p(attn, p):
    from online_softmax_streaming_amd import _lib
    g = 1 << 24
    rc = _lib.lib().attn_fwd_dropout(g, 2 * g, 3 * g, 4 * g, 1, 2, 2, 64, 64, 64, 0, 0.125, p, 1, 0,
                                     2, None, None, None)
    assert rc == 1, _lib.lib().attn_last_error()


# --------------------------------------------------------------------------
# Dispatch checks for the host-only sanitizer build (test_host_sanitizer.py):
# every entry point driven past validation into its path selection, split
# planning and launch with placeholder device addresses.  They run only
# against that build, whose HIP stand-ins fail every device call (so each
# call ends in ATTN_E_HIP and nothing is ever launched); with the real
# library they are skipped.

_SANITIZER_BUILD = (os.environ.get("ATTN_HOST_SANITIZER") == "1"
                    and "hostsan" in os.environ.get("ATTN_LIB_PATH", ""))
sanitizer_only = pytest.mark.skipif(not _SANITIZER_BUILD,
                                    reason="host-only sanitizer build not loaded")


def _ptrs(n):
    # Well-separated, 16-byte-aligned placeholder addresses (1 TiB apart), so
    # no overlap check fires; nothing dereferences them in this build.
    import ctypes
    return [ctypes.c_void_p((i + 1) << 40) for i in range(n)]


@sanitizer_only
@pytest.mark.parametrize("b,h,nq,nk,d,causal,dtype", [
    (2, 4, 1024, 1024, 64, 1, 2),      # small: keys split over waves
    (4, 16, 4096, 4096, 128, 1, 2),    # headline: tiled prefill
    (3, 8, 4099, 4099, 64, 0, 1),      # ragged fp16
    (1, 1, 128, 128, 64, 0, 0),        # FP32 vector-ALU prefill
    (16, 32, 1, 32768, 128, 0, 2),     # decode: split plan + scratch
    (2, 4, 17, 9000, 128, 1, 2),       # mid-row decode route
    (2, 4, 5, 0, 32, 1, 2),            # Nk = 0: fill kernel
])
def test_dispatch_attn_fwd(attn, b, h, nq, nk, d, causal, dtype):
    from online_softmax_streaming_amd import _lib
    q, k, v, o, m, l = _ptrs(6)
    L = _lib.lib()
    assert L.attn_fwd(q, k, v, o, b, h, nq, nk, d, causal, 0.125, dtype, None) == attn.ATTN_E_HIP
    assert L.attn_fwd_stats(q, k, v, o, b, h, nq, nk, d, causal, 0.125, dtype, m, l,
                            None) == attn.ATTN_E_HIP
    assert L.attn_fwd_gqa(q, k, v, o, b, h, 1 if h % 2 else 2, nq, nk, d, causal, 0.125, dtype,
                          m, l, None) == attn.ATTN_E_HIP


@sanitizer_only
def test_dispatch_variants(attn):
    from online_softmax_streaming_amd import _lib
    L = _lib.lib()
    q, k, v, o, m, l, mask, do, dq, dk, dv, t, lens = _ptrs(13)
    E = attn.ATTN_E_HIP
    assert L.attn_fwd_masked(q, k, v, o, mask, 1 << 20, 1 << 16, 2, 4, 2, 300, 300, 64, 1, 100,
                             0.125, 2, m, l, None) == E
    assert L.attn_fwd_masked(q, k, v, o, None, 0, 0, 2, 4, 4, 300, 300, 64, 1, 100, 0.125, 1,
                             None, None, None) == E
    assert L.attn_fwd_dropout(q, k, v, o, 2, 4, 2, 300, 300, 128, 1, 0.125, 0.1, 7, 0, 2, m, l,
                              None) == E
    assert L.attn_fwd_varlen(q, k, v, o, t, lens, 4, 8, 2, 5000, 6000, 2000, 64, 1, 0.125, 2, m,
                             l, None) == E
    for dtype in (0, 1, 2):
        assert L.attn_bwd(q, k, v, o, do, m, l, dq, dk, dv, 2, 4, 2, 500, 700, 64, 1, 0.125,
                          dtype, None) == E
    for nq, hkv in ((1, 8), (4, 2), (1, 1)):
        for fn in (L.attn_decode_paged, L.attn_decode_paged_noalloc):
            assert fn(q, k, v, t, lens, o, 4, 8, hkv, nq, 128, 512, 16, 128, 1, 0, 0.125, 2, m,
                      l, None) == E
    assert L.softmax_rows(q, o, 1024, 131072, 0, 2, None) == E
    assert L.softmax_rows(q, o, 3, 1001, 256, 1, None) == E
    assert L.softmax_rows_scratch_bytes(4, 32769, 1024) == 1088
    assert L.online_merge_batch(q, k, v, o, m, l, 1000, None) == E
    assert b"no device" in L.attn_last_error()
