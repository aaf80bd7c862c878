"""ctypes view of the C ABI declared in include/attn.h.

Loading fails loudly when the HIP library has not been built: there is no
fallback path.
"""
from __future__ import annotations

import ctypes
import pathlib

LIB_PATH = pathlib.Path(__file__).resolve().parent / "libattn_mi355x.so"


class Strides(ctypes.Structure):
    """attn_strides_t: element strides {batch, token, head} of q, k, v, o."""
    _fields_ = [("q", ctypes.c_int64 * 3), ("k", ctypes.c_int64 * 3),
                ("v", ctypes.c_int64 * 3), ("o", ctypes.c_int64 * 3)]


class PagedKv(ctypes.Structure):
    """attn_paged_kv_t: page table, sequence lengths and element strides of a paged KV cache."""
    _fields_ = [("block_table", ctypes.c_void_p), ("seq_lens", ctypes.c_void_p), ("num_blocks", ctypes.c_int),
                ("block_size", ctypes.c_int), ("max_blocks", ctypes.c_int), ("page_stride", ctypes.c_int64),
                ("token_stride", ctypes.c_int64), ("head_stride", ctypes.c_int64)]


SYMBOLS = {
    # name: (restype, argtypes)
    "attn_fwd": (ctypes.c_int, [ctypes.c_void_p] * 4 + [ctypes.c_void_p] + [ctypes.c_int] * 7
                 + [ctypes.c_float, ctypes.c_int, ctypes.c_void_p]),
    "attn_fwd_strided": (ctypes.c_int, [ctypes.c_void_p] * 4 + [ctypes.c_void_p] + [ctypes.c_int] * 7
                         + [ctypes.c_float, ctypes.c_int, ctypes.POINTER(Strides), ctypes.c_void_p]),
    "attn_fwd_fp8qk": (ctypes.c_int, [ctypes.c_void_p] * 5 + [ctypes.c_float] * 2 + [ctypes.c_int] * 7
                       + [ctypes.c_float, ctypes.c_int, ctypes.c_void_p]),
    "attn_decode_workspace_bytes": (ctypes.c_size_t, [ctypes.c_int] * 5),
    "attn_decode_splitkv": (ctypes.c_int, [ctypes.c_void_p] * 5 + [ctypes.c_int] * 6
                            + [ctypes.c_float, ctypes.c_int, ctypes.c_void_p]),
    "attn_decode_paged_splitkv": (ctypes.c_int, [ctypes.c_void_p] * 3 + [ctypes.POINTER(PagedKv)]
                                  + [ctypes.c_void_p] * 2 + [ctypes.c_int] * 5
                                  + [ctypes.c_float, ctypes.c_int, ctypes.c_void_p]),
    "attn_decode_paged_fp8kv_splitkv": (ctypes.c_int, [ctypes.c_void_p] * 3 + [ctypes.c_float] * 2
                                        + [ctypes.POINTER(PagedKv)] + [ctypes.c_void_p] * 2 + [ctypes.c_int] * 5
                                        + [ctypes.c_float, ctypes.c_int, ctypes.c_void_p]),
    "attn_decode_fp8kv_splitkv": (ctypes.c_int, [ctypes.c_void_p] * 3 + [ctypes.c_float] * 2 + [ctypes.c_void_p] * 2
                                  + [ctypes.c_int] * 6 + [ctypes.c_float, ctypes.c_int, ctypes.c_void_p]),
    "attn_decode_fused_workspace_bytes": (ctypes.c_size_t, [ctypes.c_int] * 5),
    "attn_decode_fused": (ctypes.c_int, [ctypes.c_void_p] * 5 + [ctypes.c_void_p, ctypes.c_size_t] + [ctypes.c_int] * 5
                          + [ctypes.c_float, ctypes.c_int, ctypes.c_void_p]),
    "attn_decode_paged_fused": (ctypes.c_int, [ctypes.c_void_p] * 3 + [ctypes.POINTER(PagedKv)] + [ctypes.c_void_p] * 3
                                + [ctypes.c_size_t] + [ctypes.c_int] * 4 + [ctypes.c_float, ctypes.c_int, ctypes.c_void_p]),
    "attn_decode_fp8kv_fused": (ctypes.c_int, [ctypes.c_void_p] * 3 + [ctypes.c_float] * 2 + [ctypes.c_void_p] * 3
                                + [ctypes.c_size_t] + [ctypes.c_int] * 5 + [ctypes.c_float, ctypes.c_int, ctypes.c_void_p]),
    "attn_decode_paged_fp8kv_fused": (ctypes.c_int, [ctypes.c_void_p] * 3 + [ctypes.c_float] * 2
                                      + [ctypes.POINTER(PagedKv)] + [ctypes.c_void_p] * 3 + [ctypes.c_size_t]
                                      + [ctypes.c_int] * 4 + [ctypes.c_float, ctypes.c_int, ctypes.c_void_p]),
    "attn_decode_fused_noalloc": (ctypes.c_int, [ctypes.c_void_p] * 5 + [ctypes.c_int] * 5
                                  + [ctypes.c_float, ctypes.c_int, ctypes.c_void_p]),
    "lse_merge": (ctypes.c_int, [ctypes.c_void_p] * 4 + [ctypes.c_int] * 4
                  + [ctypes.c_int, ctypes.c_void_p]),
    "attn_status_string": (ctypes.c_char_p, [ctypes.c_int]),
}

_lib = None


def load() -> ctypes.CDLL:
    """The loaded library (raises if it is missing)."""
    global _lib
    if _lib is None:
        if not LIB_PATH.exists():
            raise RuntimeError(
                f"{LIB_PATH.name} is not built; run `python -m attention_attn_fwd_06_amd.build` "
                "(or __graft_entry__.build()) first")
        lib = ctypes.CDLL(str(LIB_PATH))
        for name, (res, args) in SYMBOLS.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib
