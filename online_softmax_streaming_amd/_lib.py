"""ctypes loader for the in-tree HIP library libattn.so.

There is no fallback: if the library has not been built, or cannot be
loaded, every call raises.  Build it with ``__graft_entry__.build()`` or
``python online_softmax_streaming_amd/build.py``.
"""

import ctypes
import os
import threading

# ATTN_LIB_PATH names another build of the same C ABI (the tests' host-only
# sanitizer build); by default the in-tree library is loaded.
LIB_PATH = os.environ.get("ATTN_LIB_PATH") or os.path.join(
    os.path.dirname(os.path.abspath(__file__)), "libattn.so")

_lock = threading.Lock()
_lib = None

_c_i64 = ctypes.c_int64
_c_ptr = ctypes.c_void_p
_c_fptr = ctypes.POINTER(ctypes.c_float)

# Exported symbols and their C signatures, as declared in include/attn.h.
SIGNATURES = {
    "attn_fwd": (ctypes.c_int, [_c_ptr, _c_ptr, _c_ptr, _c_ptr, _c_i64, _c_i64, _c_i64, _c_i64,
                                _c_i64, ctypes.c_int, ctypes.c_float, ctypes.c_int, _c_ptr]),
    "attn_fwd_stats": (ctypes.c_int, [_c_ptr, _c_ptr, _c_ptr, _c_ptr, _c_i64, _c_i64, _c_i64,
                                      _c_i64, _c_i64, ctypes.c_int, ctypes.c_float, ctypes.c_int,
                                      _c_ptr, _c_ptr, _c_ptr]),
    "attn_fwd_gqa": (ctypes.c_int, [_c_ptr, _c_ptr, _c_ptr, _c_ptr, _c_i64, _c_i64, _c_i64, _c_i64,
                                    _c_i64, _c_i64, ctypes.c_int, ctypes.c_float, ctypes.c_int,
                                    _c_ptr, _c_ptr, _c_ptr]),
    "attn_bwd": (ctypes.c_int, [_c_ptr] * 10 + [_c_i64] * 6 + [ctypes.c_int, ctypes.c_float,
                                                                 ctypes.c_int, _c_ptr]),
    "attn_decode_paged": (ctypes.c_int, [_c_ptr] * 6 + [_c_i64] * 8 + [ctypes.c_int, _c_i64,
                                                                       ctypes.c_float, ctypes.c_int,
                                                                       _c_ptr, _c_ptr, _c_ptr]),
    "attn_decode_paged_noalloc": (ctypes.c_int, [_c_ptr] * 6 + [_c_i64] * 8 + [ctypes.c_int, _c_i64,
                                                                               ctypes.c_float, ctypes.c_int,
                                                                               _c_ptr, _c_ptr, _c_ptr]),
    "attn_fwd_varlen": (ctypes.c_int, [_c_ptr] * 6 + [_c_i64] * 7 + [ctypes.c_int, ctypes.c_float,
                                                                     ctypes.c_int, _c_ptr, _c_ptr,
                                                                     _c_ptr]),
    "attn_fwd_masked": (ctypes.c_int, [_c_ptr] * 5 + [_c_i64] * 8 + [ctypes.c_int, _c_i64,
                                                                     ctypes.c_float, ctypes.c_int,
                                                                     _c_ptr, _c_ptr, _c_ptr]),
    "attn_fwd_dropout": (ctypes.c_int, [_c_ptr] * 4 + [_c_i64] * 6 + [ctypes.c_int, ctypes.c_float,
                                                                      ctypes.c_float, ctypes.c_uint64,
                                                                      ctypes.c_uint64, ctypes.c_int,
                                                                      _c_ptr, _c_ptr, _c_ptr]),
    "online_merge": (ctypes.c_int, [ctypes.c_double, ctypes.c_double, ctypes.c_double,
                                    ctypes.c_double, ctypes.POINTER(ctypes.c_double),
                                    ctypes.POINTER(ctypes.c_double)]),
    "online_merge_batch": (ctypes.c_int, [_c_ptr, _c_ptr, _c_ptr, _c_ptr, _c_ptr, _c_ptr, _c_i64,
                                          _c_ptr]),
    "softmax_rows": (ctypes.c_int, [_c_ptr, _c_ptr, _c_i64, _c_i64, _c_i64, ctypes.c_int, _c_ptr]),
    "softmax_rows_scratch_bytes": (_c_i64, [_c_i64, _c_i64, _c_i64]),
    "attn_strerror": (ctypes.c_char_p, [ctypes.c_int]),
    "attn_last_error": (ctypes.c_char_p, []),
}


def lib():
    """The loaded library (loaded once per process)."""
    global _lib
    if _lib is not None:
        return _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise RuntimeError(
                    f"HIP library {LIB_PATH} is not built; run __graft_entry__.build()")
            handle = ctypes.CDLL(LIB_PATH)
            for name, (res, args) in SIGNATURES.items():
                fn = getattr(handle, name)
                fn.restype = res
                fn.argtypes = args
            _lib = handle
    return _lib
