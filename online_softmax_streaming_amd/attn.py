"""Python binding of the C ABI in include/attn.h (argument marshalling only).

Tensors are PyTorch device tensors: torch supplies the memory and the
stream, and every step of the computation runs in the HIP kernels of
libattn.so.  Nothing here computes attention; there is no CPU path.
"""

import contextlib
import ctypes
import math

import torch

from ._lib import lib

ATTN_F32, ATTN_F16, ATTN_BF16 = 0, 1, 2
ATTN_OK, ATTN_E_INVALID, ATTN_E_UNSUPPORTED, ATTN_E_HIP = 0, 1, 2, 3

_DTYPES = {torch.float32: ATTN_F32, torch.float16: ATTN_F16, torch.bfloat16: ATTN_BF16}

class AttnError(RuntimeError):
    """A non-zero status from the library."""

    def __init__(self, code, where):
        self.code = code
        detail = lib().attn_last_error().decode()
        super().__init__(f"{where}: {attn_strerror(code)} ({code})" + (f": {detail}" if detail else ""))


def attn_strerror(code):
    """Text for a status code."""
    return lib().attn_strerror(int(code)).decode()


def _check(rc, where):
    if rc != ATTN_OK:
        raise AttnError(rc, where)


def default_scale(d):
    """1/sqrt(D) rounded to FP32, the scale the pages use."""
    return float(torch.tensor(1.0 / math.sqrt(d), dtype=torch.float32))


def _stream_handle(stream, device):
    """The HIP stream to queue on: ``stream``, else torch's current stream of
    ``device`` (a torch.device or an index)."""
    if stream is None:
        idx = device if isinstance(device, int) else device.index
        return ctypes.c_void_p(torch._C._cuda_getCurrentRawStream(idx))
    return ctypes.c_void_p(stream.cuda_stream)


_NO_SWITCH = contextlib.nullcontext()


def _on_device(t):
    """Makes t's GPU current for the call (nothing to do when it already is)."""
    idx = t.get_device()
    return _NO_SWITCH if idx == torch.cuda.current_device() else torch.cuda.device(idx)


def _validate(q, k, v, grouped=False):
    # Common case first, with few tensor attribute reads; anything it does
    # not accept goes through the checks below, which name the problem.
    try:
        dt = q.dtype
        ok = (dt in _DTYPES and dt == k.dtype == v.dtype and q.is_cuda and k.is_cuda
              and v.is_cuda and q.dim() == 4 and k.dim() == 4 and v.dim() == 4
              and q.is_contiguous() and k.is_contiguous() and v.is_contiguous()
              and q.get_device() == k.get_device() == v.get_device())
    except AttributeError:
        ok = False
    if ok:
        qs, ks = q.shape, k.shape
        if (ks == v.shape and ks[0] == qs[0] and ks[3] == qs[3]
                and (ks[1] >= 1 and qs[1] % ks[1] == 0 if grouped else ks[1] == qs[1])):
            return
    _validate_slow(q, k, v, grouped)


def _validate_slow(q, k, v, grouped):
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name} must be a torch.Tensor")
        if t.device.type != "cuda":
            raise ValueError(f"{name} must be a GPU tensor (got {t.device}); there is no CPU path")
        if t.dim() != 4:
            raise ValueError(f"{name} must be 4-D [B, H, N, D], got shape {tuple(t.shape)}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        if t.dtype not in _DTYPES:
            raise ValueError(f"{name} has unsupported dtype {t.dtype}")
    if not (q.dtype == k.dtype == v.dtype):
        raise ValueError("q, k and v must share one dtype")
    if not (q.device == k.device == v.device):
        raise ValueError("q, k and v must be on one device")
    if k.shape != v.shape:
        raise ValueError(f"k and v shapes differ: {tuple(k.shape)} vs {tuple(v.shape)}")
    b, h, _, d = q.shape
    if grouped:
        hkv = k.shape[1]
        if (k.shape[0], k.shape[3]) != (b, d) or hkv < 1 or h % hkv:
            raise ValueError(f"q {tuple(q.shape)} and k {tuple(k.shape)}: need equal B and D "
                             "and K/V heads dividing the query heads")
    elif (k.shape[0], k.shape[1], k.shape[3]) != (b, h, d):
        raise ValueError(f"q {tuple(q.shape)} and k {tuple(k.shape)} disagree on B, H or D")


def attn_fwd_stats(q, k, v, causal=False, scale=None, out=None, m_out=None, l_out=None,
                   stream=None, want_stats=True, _grouped=False):
    """Streaming attention forward; returns (out, m, l).

    q: [B, H, Nq, D]; k, v: [B, H, Nk, D]; one dtype (float32, float16 or
    bfloat16), contiguous, on one GPU.  ``out`` (same shape/dtype as q) and
    the float32 [B, H, Nq] arrays ``m_out`` / ``l_out`` are allocated when not
    given.  ``scale`` defaults to FP32(1/sqrt(D)).  The work is queued on
    ``stream`` (default: torch's current stream of q's device).
    """
    _validate(q, k, v, grouped=_grouped)
    b, h, nq, d = q.shape
    nk = k.shape[2]
    if scale is None:
        scale = default_scale(d)
    if out is None:
        out = torch.empty_like(q)
    elif (out.shape != q.shape or out.dtype != q.dtype or not out.is_cuda
          or out.get_device() != q.get_device() or not out.is_contiguous()):
        raise ValueError("out must be a contiguous tensor like q")
    if want_stats:
        for name, t in (("m_out", m_out), ("l_out", l_out)):
            if t is not None and (t.dtype != torch.float32 or t.device != q.device
                                  or t.shape != (b, h, nq) or not t.is_contiguous()):
                raise ValueError(f"{name} must be a contiguous float32 [B, H, Nq] GPU tensor")
        if m_out is None:
            m_out = torch.empty((b, h, nq), dtype=torch.float32, device=q.device)
        if l_out is None:
            l_out = torch.empty((b, h, nq), dtype=torch.float32, device=q.device)
    with _on_device(q):
        sh = _stream_handle(stream, q.get_device())
        args = (ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(k.data_ptr()),
                ctypes.c_void_p(v.data_ptr()), ctypes.c_void_p(out.data_ptr()),
                b, h, nq, nk, d, int(bool(causal)), float(scale), _DTYPES[q.dtype])
        if _grouped:
            gargs = args[:6] + (k.shape[1],) + args[6:]
            stats = ((ctypes.c_void_p(m_out.data_ptr()), ctypes.c_void_p(l_out.data_ptr()))
                     if want_stats else (None, None))
            _check(lib().attn_fwd_gqa(*gargs, *stats, sh), "attn_fwd_gqa")
        elif want_stats:
            rc = lib().attn_fwd_stats(*args, ctypes.c_void_p(m_out.data_ptr()),
                                      ctypes.c_void_p(l_out.data_ptr()), sh)
            _check(rc, "attn_fwd_stats")
        else:
            _check(lib().attn_fwd(*args, sh), "attn_fwd")
    return out, m_out, l_out


def attn_fwd_gqa(q, k, v, causal=False, scale=None, out=None, m_out=None, l_out=None,
                 stream=None, want_stats=False):
    """Grouped-query attention forward: k, v are [B, Hkv, Nk, D] with Hkv
    dividing H, and query head h attends with K/V head h // (H // Hkv).
    Returns (out, m, l); m and l are None unless ``want_stats``."""
    return attn_fwd_stats(q, k, v, causal=causal, scale=scale, out=out, m_out=m_out,
                          l_out=l_out, stream=stream, want_stats=want_stats, _grouped=True)


def attn_fwd(q, k, v, causal=False, scale=None, out=None, stream=None):
    """Streaming attention forward; returns ``out`` [B, H, Nq, D]."""
    return attn_fwd_stats(q, k, v, causal=causal, scale=scale, out=out, stream=stream,
                          want_stats=False)[0]


def attn_bwd(q, k, v, out, dout, m, l, causal=False, scale=None, dq=None, dk=None, dv=None,
             stream=None):
    """Attention backward; returns (dq, dk, dv).

    q, out, dout: [B, H, Nq, D]; k, v: [B, Hkv, Nk, D] (Hkv dividing H);
    float16 or bfloat16, contiguous, on one GPU.  ``out``, ``m`` and ``l``
    are what attn_fwd_stats / attn_fwd_gqa returned for the same inputs
    (m, l: float32 [B, H, Nq]).  ``scale`` defaults to FP32(1/sqrt(D)) and
    must be the forward's.  Outputs are allocated when not given.
    """
    _validate(q, k, v, grouped=True)
    b, h, nq, d = q.shape
    hkv, nk = k.shape[1], k.shape[2]
    for name, t in (("out", out), ("dout", dout)):
        if (not isinstance(t, torch.Tensor) or t.shape != q.shape or t.dtype != q.dtype
                or t.device != q.device or not t.is_contiguous()):
            raise ValueError(f"{name} must be a contiguous tensor like q")
    for name, t in (("m", m), ("l", l)):
        if (not isinstance(t, torch.Tensor) or t.dtype != torch.float32 or t.device != q.device
                or t.shape != (b, h, nq) or not t.is_contiguous()):
            raise ValueError(f"{name} must be a contiguous float32 [B, H, Nq] GPU tensor")
    if scale is None:
        scale = default_scale(d)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    for name, t, like in (("dq", dq, q), ("dk", dk, k), ("dv", dv, v)):
        if (t.shape != like.shape or t.dtype != like.dtype or t.device != like.device
                or not t.is_contiguous()):
            raise ValueError(f"{name} must be a contiguous tensor like {'q' if like is q else 'k'}")
    with _on_device(q):
        sh = _stream_handle(stream, q.get_device())
        ptrs = (ctypes.c_void_p(t.data_ptr()) for t in (q, k, v, out, dout, m, l, dq, dk, dv))
        rc = lib().attn_bwd(*ptrs, b, h, hkv, nq, nk, d, int(bool(causal)), float(scale),
                            _DTYPES[q.dtype], sh)
    _check(rc, "attn_bwd")
    return dq, dk, dv


def pack_mask(mask):
    """Bit-pack a bool tensor [..., Nq, Nk] into int32 words [..., Nq,
    ceil(Nk/32)] (bit j % 32 of word j / 32), the layout attn_fwd_masked
    reads.  Input marshalling only; runs where ``mask`` lives."""
    if not isinstance(mask, torch.Tensor) or mask.dtype != torch.bool:
        raise ValueError("mask must be a bool tensor")
    nk = mask.shape[-1]
    words = (nk + 31) // 32
    pad = words * 32 - nk
    m = torch.nn.functional.pad(mask.to(torch.int64), (0, pad))
    m = m.reshape(*mask.shape[:-1], words, 32)
    weights = torch.tensor([1 << i for i in range(32)], dtype=torch.int64, device=mask.device)
    packed = (m * weights).sum(dim=-1)
    return torch.where(packed >= 1 << 31, packed - (1 << 32), packed).to(torch.int32).contiguous()


def attn_fwd_masked(q, k, v, mask=None, causal=False, window=0, scale=None, out=None,
                    want_stats=False, stream=None):
    """Attention with an arbitrary mask and/or a sliding window; returns
    (out, m, l) (m, l None unless ``want_stats``).

    q: [B, H, Nq, D]; k, v: [B, Hkv, Nk, D].  ``mask``: None, or packed
    int32 words [Bm, Hm, Nq, ceil(Nk/32)] with Bm in {1, B} and Hm in {1, H}
    (see pack_mask); a size-1 dimension broadcasts.  ``window`` > 0 keeps
    the last ``window`` keys up to each row's diagonal (needs ``causal``).
    """
    _validate(q, k, v, grouped=True)
    b, h, nq, d = q.shape
    hkv, nk = k.shape[1], k.shape[2]
    sb = sh = 0
    if mask is not None:
        words = (nk + 31) // 32
        if (not isinstance(mask, torch.Tensor) or mask.dtype != torch.int32
                or mask.device != q.device or not mask.is_contiguous() or mask.dim() != 4
                or tuple(mask.shape[2:]) != (nq, words) or mask.shape[0] not in (1, b)
                or mask.shape[1] not in (1, h)):
            raise ValueError("mask must be contiguous int32 [B or 1, H or 1, Nq, ceil(Nk/32)] "
                             "on q's device")
        sh = nq * words if mask.shape[1] == h else 0
        sb = mask.shape[1] * nq * words if mask.shape[0] == b else 0
    if scale is None:
        scale = default_scale(d)
    if out is None:
        out = torch.empty_like(q)
    elif (out.shape != q.shape or out.dtype != q.dtype or not out.is_cuda
          or out.get_device() != q.get_device() or not out.is_contiguous()):
        raise ValueError("out must be a contiguous tensor like q")
    m = l = None
    if want_stats:
        m = torch.empty((b, h, nq), dtype=torch.float32, device=q.device)
        l = torch.empty((b, h, nq), dtype=torch.float32, device=q.device)
    with _on_device(q):
        sth = _stream_handle(stream, q.get_device())
        rc = lib().attn_fwd_masked(
            *(ctypes.c_void_p(t.data_ptr()) for t in (q, k, v, out)),
            ctypes.c_void_p(mask.data_ptr()) if mask is not None else None, sb, sh,
            b, h, hkv, nq, nk, d, int(bool(causal)), int(window), float(scale), _DTYPES[q.dtype],
            ctypes.c_void_p(m.data_ptr()) if want_stats else None,
            ctypes.c_void_p(l.data_ptr()) if want_stats else None, sth)
    _check(rc, "attn_fwd_masked")
    return out, m, l


def attn_fwd_dropout(q, k, v, p, seed, offset=0, causal=False, scale=None, out=None,
                     want_stats=False, stream=None):
    """Attention with dropout on the probabilities (Philox4x64-10 keep mask,
    kept weights scaled by 65536 / (65536 - round(p * 65536))); returns
    (out, m, l) (m, l None unless ``want_stats``).  q: [B, H, Nq, D];
    k, v: [B, Hkv, Nk, D]."""
    _validate(q, k, v, grouped=True)
    b, h, nq, d = q.shape
    hkv, nk = k.shape[1], k.shape[2]
    if scale is None:
        scale = default_scale(d)
    if out is None:
        out = torch.empty_like(q)
    elif (out.shape != q.shape or out.dtype != q.dtype or not out.is_cuda
          or out.get_device() != q.get_device() or not out.is_contiguous()):
        raise ValueError("out must be a contiguous tensor like q")
    m = l = None
    if want_stats:
        m = torch.empty((b, h, nq), dtype=torch.float32, device=q.device)
        l = torch.empty((b, h, nq), dtype=torch.float32, device=q.device)
    with _on_device(q):
        sth = _stream_handle(stream, q.get_device())
        rc = lib().attn_fwd_dropout(
            *(ctypes.c_void_p(t.data_ptr()) for t in (q, k, v, out)), b, h, hkv, nq, nk, d,
            int(bool(causal)), float(scale), float(p), int(seed), int(offset), _DTYPES[q.dtype],
            ctypes.c_void_p(m.data_ptr()) if want_stats else None,
            ctypes.c_void_p(l.data_ptr()) if want_stats else None, sth)
    _check(rc, "attn_fwd_dropout")
    return out, m, l


def attn_fwd_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q=None, causal=False,
                    scale=None, out=None, want_stats=False, stream=None):
    """Attention over packed sequences of different lengths; returns
    (out, m, l) (m, l None unless ``want_stats``; head-major [H, total_q]).

    q: [total_q, H, D]; k, v: [total_k, Hkv, D] (Hkv dividing H); one
    dtype, contiguous, on one GPU.  cu_seqlens_q / cu_seqlens_k: int32
    [B + 1] offsets of each sequence's first row.  ``max_seqlen_q``: the
    longest query sequence; when None it is read from cu_seqlens_q, which
    synchronises the host with the device.
    """
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not isinstance(t, torch.Tensor) or t.device.type != "cuda" or t.dim() != 3:
            raise ValueError(f"{name} must be a 3-D GPU tensor [total, heads, D]")
        if not t.is_contiguous() or t.dtype not in _DTYPES or t.dtype != q.dtype:
            raise ValueError(f"{name} must be contiguous and share q's dtype")
    if k.shape != v.shape or k.shape[2] != q.shape[2]:
        raise ValueError("k and v must match and share q's D")
    total_q, h, d = q.shape
    total_k, hkv, _ = k.shape
    for name, t in (("cu_seqlens_q", cu_seqlens_q), ("cu_seqlens_k", cu_seqlens_k)):
        if (not isinstance(t, torch.Tensor) or t.dtype != torch.int32 or t.device != q.device
                or t.dim() != 1 or not t.is_contiguous()):
            raise ValueError(f"{name} must be a contiguous int32 1-D GPU tensor")
    if cu_seqlens_q.shape != cu_seqlens_k.shape or cu_seqlens_q.shape[0] < 1:
        raise ValueError("cu_seqlens_q and cu_seqlens_k must both be [B + 1]")
    b = cu_seqlens_q.shape[0] - 1
    if max_seqlen_q is None:
        max_seqlen_q = int((cu_seqlens_q[1:] - cu_seqlens_q[:-1]).max().item()) if b else 0
    if scale is None:
        scale = default_scale(d)
    if out is None:
        out = torch.empty_like(q)
    elif (out.shape != q.shape or out.dtype != q.dtype or not out.is_cuda
          or out.get_device() != q.get_device() or not out.is_contiguous()):
        raise ValueError("out must be a contiguous tensor like q")
    m = l = None
    if want_stats:
        m = torch.empty((h, total_q), dtype=torch.float32, device=q.device)
        l = torch.empty((h, total_q), dtype=torch.float32, device=q.device)
    with _on_device(q):
        sh = _stream_handle(stream, q.get_device())
        stats = ((ctypes.c_void_p(m.data_ptr()), ctypes.c_void_p(l.data_ptr()))
                 if want_stats else (None, None))
        rc = lib().attn_fwd_varlen(
            *(ctypes.c_void_p(t.data_ptr()) for t in (q, k, v, out, cu_seqlens_q, cu_seqlens_k)),
            b, h, hkv, total_q, total_k, int(max_seqlen_q), d, int(bool(causal)), float(scale),
            _DTYPES[q.dtype], *stats, sh)
    _check(rc, "attn_fwd_varlen")
    return out, m, l


def attn_decode_paged_noalloc(q, k_cache, v_cache, block_table, seq_lens, causal=True,
                              window=0, scale=None, out=None, m_out=None, l_out=None,
                              want_stats=False, stream=None):
    """attn_decode_paged through the entry point that allocates nothing
    (the key splits' partial states go to a fixed 4 MiB device buffer per
    GPU; calls that may overlap on one GPU race on it).  Pass ``out`` (and
    ``m_out``/``l_out``) to keep the call itself free of allocations."""
    return attn_decode_paged(q, k_cache, v_cache, block_table, seq_lens, causal=causal,
                             window=window, scale=scale, out=out, m_out=m_out, l_out=l_out,
                             want_stats=want_stats, stream=stream, _entry="attn_decode_paged_noalloc")


def attn_decode_paged(q, k_cache, v_cache, block_table, seq_lens, causal=True, window=0,
                      scale=None, out=None, m_out=None, l_out=None, want_stats=False,
                      stream=None, _entry="attn_decode_paged"):
    """Attention over a paged K/V cache; returns (out, m, l) (m, l None
    unless ``want_stats``).

    q: [B, H, Nq, D]; k_cache, v_cache: [num_pages, Hkv, page_size, D]
    (Hkv dividing H, page_size a power of two); block_table: int32
    [B, max_pages] of physical page indices; seq_lens: int32 [B] key counts.
    ``window`` > 0 keeps the last ``window`` keys up to each row's diagonal
    (needs ``causal``).
    """
    for name, t in (("q", q), ("k_cache", k_cache), ("v_cache", v_cache)):
        if not isinstance(t, torch.Tensor) or t.device.type != "cuda" or t.dim() != 4:
            raise ValueError(f"{name} must be a 4-D GPU tensor")
        if not t.is_contiguous() or t.dtype not in _DTYPES or t.dtype != q.dtype:
            raise ValueError(f"{name} must be contiguous and share q's dtype")
    if k_cache.shape != v_cache.shape:
        raise ValueError("k_cache and v_cache shapes differ")
    b, h, nq, d = q.shape
    num_pages, hkv, page_size, dk = k_cache.shape
    if dk != d:
        raise ValueError("q and the caches disagree on D")
    for name, t in (("block_table", block_table), ("seq_lens", seq_lens)):
        if (not isinstance(t, torch.Tensor) or t.dtype != torch.int32 or t.device != q.device
                or not t.is_contiguous()):
            raise ValueError(f"{name} must be a contiguous int32 GPU tensor")
    if block_table.dim() != 2 or block_table.shape[0] != b or seq_lens.shape != (b,):
        raise ValueError("block_table must be [B, max_pages] and seq_lens [B]")
    max_pages = block_table.shape[1]
    if scale is None:
        scale = default_scale(d)
    if out is None:
        out = torch.empty_like(q)
    elif (out.shape != q.shape or out.dtype != q.dtype or not out.is_cuda
          or out.get_device() != q.get_device() or not out.is_contiguous()):
        raise ValueError("out must be a contiguous tensor like q")
    if want_stats:
        m_out = torch.empty((b, h, nq), dtype=torch.float32, device=q.device) if m_out is None else m_out
        l_out = torch.empty((b, h, nq), dtype=torch.float32, device=q.device) if l_out is None else l_out
        for name, t in (("m_out", m_out), ("l_out", l_out)):
            if (t.dtype != torch.float32 or t.device != q.device or t.shape != (b, h, nq)
                    or not t.is_contiguous()):
                raise ValueError(f"{name} must be a contiguous float32 [B, H, Nq] GPU tensor")
    with _on_device(q):
        sh = _stream_handle(stream, q.get_device())
        stats = ((ctypes.c_void_p(m_out.data_ptr()), ctypes.c_void_p(l_out.data_ptr()))
                 if want_stats else (None, None))
        rc = getattr(lib(), _entry)(
            *(ctypes.c_void_p(t.data_ptr()) for t in (q, k_cache, v_cache, block_table, seq_lens,
                                                      out)),
            b, h, hkv, nq, d, num_pages, page_size, max_pages, int(bool(causal)), int(window),
            float(scale), _DTYPES[q.dtype], *stats, sh)
    _check(rc, _entry)
    return out, (m_out if want_stats else None), (l_out if want_stats else None)


def attn_fwd_raw(q_ptr, k_ptr, v_ptr, out_ptr, b, h, nq, nk, d, causal, scale, dtype,
                 stream_handle=0):
    """Direct C call with raw device pointers; returns the status code."""
    return lib().attn_fwd(ctypes.c_void_p(q_ptr), ctypes.c_void_p(k_ptr), ctypes.c_void_p(v_ptr),
                          ctypes.c_void_p(out_ptr), b, h, nq, nk, d, int(causal), float(scale),
                          int(dtype), ctypes.c_void_p(stream_handle))


def online_merge(m1, l1, m2, l2):
    """Host A1 merge in double precision; returns (m, l)."""
    m = ctypes.c_double()
    l = ctypes.c_double()
    _check(lib().online_merge(float(m1), float(l1), float(m2), float(l2), ctypes.byref(m),
                              ctypes.byref(l)), "online_merge")
    return m.value, l.value


def online_merge_batch(m1, l1, m2, l2, m=None, l=None, stream=None):
    """Elementwise A1 merge of float32 GPU tensors of one shape; returns (m, l)."""
    ts = (m1, l1, m2, l2)
    for t in ts:
        if (not isinstance(t, torch.Tensor) or t.device.type != "cuda"
                or t.dtype != torch.float32 or not t.is_contiguous() or t.shape != m1.shape
                or t.device != m1.device):
            raise ValueError("online_merge_batch takes contiguous float32 GPU tensors of one shape")
    m = torch.empty_like(m1) if m is None else m
    l = torch.empty_like(m1) if l is None else l
    for t in (m, l):
        if t.shape != m1.shape or t.dtype != torch.float32 or not t.is_contiguous():
            raise ValueError("outputs must be contiguous float32 tensors like the inputs")
    with _on_device(m1):
        sh = _stream_handle(stream, m1.get_device())
        rc = lib().online_merge_batch(*(ctypes.c_void_p(t.data_ptr()) for t in (*ts, m, l)),
                                      m1.numel(), sh)
    _check(rc, "online_merge_batch")
    return m, l


def softmax_rows(x, chunk=0, out=None, stream=None):
    """Row softmax of a contiguous 2D GPU tensor by the split method.

    Three kernels on the stream (per-chunk partial states, their A1 merge per
    row, a normalising re-read); `chunk` is 256/512/1024/2048/4096 columns or
    0 for the library's choice.  `out` may be `x` itself (in place).
    """
    if not isinstance(x, torch.Tensor) or x.device.type != "cuda":
        raise ValueError("x must be a GPU tensor; there is no CPU path")
    if x.dim() != 2 or not x.is_contiguous():
        raise ValueError("x must be a contiguous 2D tensor [M, N]")
    if x.dtype not in _DTYPES:
        raise ValueError(f"unsupported dtype {x.dtype}")
    if out is None:
        out = torch.empty_like(x)
    elif (out.shape != x.shape or out.dtype != x.dtype or out.device != x.device
          or not out.is_contiguous()):
        raise ValueError("out must be a contiguous tensor like x")
    with _on_device(x):
        sh = _stream_handle(stream, x.get_device())
        rc = lib().softmax_rows(ctypes.c_void_p(x.data_ptr()), ctypes.c_void_p(out.data_ptr()),
                                x.shape[0], x.shape[1], int(chunk), _DTYPES[x.dtype], sh)
    _check(rc, "softmax_rows")
    return out


def softmax_rows_scratch_bytes(m, n, chunk=0):
    """Scratch bytes softmax_rows takes for [m, n] (-1 for invalid sizes)."""
    return int(lib().softmax_rows_scratch_bytes(int(m), int(n), int(chunk)))
