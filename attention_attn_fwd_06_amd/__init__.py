"""MI355X (gfx950) fused attention forward and split-KV decode.

Thin Python binding over the C ABI in ``include/attn.h``: it only marshals
torch tensors (device memory and the current stream) into pointers and sizes;
every step of the computation runs in the HIP kernels of ``csrc/``.
"""
from __future__ import annotations

import ctypes

import torch

from . import _lib

__all__ = [
    "AttnError", "ATTN_F16", "ATTN_BF16", "attn_fwd", "attn_decode_splitkv", "lse_merge",
    "attn_decode_workspace_bytes", "attn_status_string", "attn_decode", "attn_decode_paged_splitkv",
    "attn_decode_paged", "attn_decode_fp8kv_splitkv", "attn_decode_fp8kv",
]

ATTN_F16 = 0
ATTN_BF16 = 1
_DTYPES = {torch.float16: ATTN_F16, torch.bfloat16: ATTN_BF16}


class AttnError(RuntimeError):
    def __init__(self, status: int, fn: str):
        super().__init__(f"{fn} failed with status {status}: {attn_status_string(status)}")
        self.status = status


def attn_status_string(status: int) -> str:
    return _lib.load().attn_status_string(int(status)).decode()


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype not in _DTYPES:
        raise TypeError(f"unsupported dtype {t.dtype}; expected float16 or bfloat16")
    return _DTYPES[t.dtype]


def _check(t: torch.Tensor, name: str):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def attn_fwd(q, k, v, causal: bool = False, scale: float | None = None, o=None, lse=None,
             return_lse: bool = True, stream=None):
    """q [B,N,Hq,d], k/v [B,M,Hkv,d] -> (o [B,N,Hq,d], lse [B,Hq,N] fp32 or None).

    q, k, v (and a given o) may be strided views (e.g. slices of a fused QKV
    projection, or head-major tensors transposed to [B,N,H,d]) as long as the
    last dimension is contiguous; they then go through attn_fwd_strided."""
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        if not t.is_cuda:
            raise ValueError(f"{n} must be a GPU tensor")
        if t.dim() != 4 or t.stride(-1) != 1:
            raise ValueError(f"{n} must be 4-D with a contiguous last dimension")
    B, N, Hq, d = q.shape
    M, Hkv = k.shape[1], k.shape[2]
    if scale is None:
        scale = d ** -0.5
    if o is None:
        o = torch.empty((B, N, Hq, d), dtype=q.dtype, device=q.device)
    elif not o.is_cuda or o.dim() != 4 or o.stride(-1) != 1:
        raise ValueError("o must be a 4-D GPU tensor with a contiguous last dimension")
    if lse is None and return_lse:
        lse = torch.empty((B, Hq, N), dtype=torch.float32, device=q.device)
    if lse is not None:
        _check(lse, "lse")
    lib = _lib.load()
    args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
            lse.data_ptr() if lse is not None else None,
            B, Hq, Hkv, N, M, d, int(bool(causal)), float(scale), _dtype_code(q))
    if all(t.is_contiguous() for t in (q, k, v, o)):
        st = lib.attn_fwd(*args, _stream(stream))
        name = "attn_fwd"
    else:
        strides = _lib.Strides()
        for field, t in (("q", q), ("k", k), ("v", v), ("o", o)):
            # the stride of a dimension of size 1 is never used: pass 0
            getattr(strides, field)[:] = [t.stride(i) if t.shape[i] > 1 else 0 for i in range(3)]
        st = lib.attn_fwd_strided(*args, ctypes.byref(strides), _stream(stream))
        name = "attn_fwd_strided"
    if st != 0:
        raise AttnError(st, name)
    return o, lse


def attn_decode_workspace_bytes(B: int, Hq: int, M: int, d: int, chunk_size: int = 128) -> int:
    return int(_lib.load().attn_decode_workspace_bytes(B, Hq, M, d, chunk_size))


def attn_decode_splitkv(q, k, v, chunk_size: int = 128, scale: float | None = None,
                        o_part=None, lse_part=None, stream=None):
    """q [B,Hq,d], k/v [B,Hkv,M,d] -> (o_part [B,Hq,C,d] fp32, lse_part [B,Hq,C] fp32)."""
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _check(t, n)
    B, Hq, d = q.shape
    Hkv, M = k.shape[1], k.shape[2]
    C = -(-M // chunk_size)
    if scale is None:
        scale = d ** -0.5
    if o_part is None:
        o_part = torch.empty((B, Hq, C, d), dtype=torch.float32, device=q.device)
    if lse_part is None:
        lse_part = torch.empty((B, Hq, C), dtype=torch.float32, device=q.device)
    st = _lib.load().attn_decode_splitkv(q.data_ptr(), k.data_ptr(), v.data_ptr(), o_part.data_ptr(),
                                         lse_part.data_ptr(), B, Hq, Hkv, M, d, chunk_size,
                                         float(scale), _dtype_code(q), _stream(stream))
    if st != 0:
        raise AttnError(st, "attn_decode_splitkv")
    return o_part, lse_part


def attn_decode_paged_splitkv(q, k_cache, v_cache, block_table, seq_lens, chunk_size: int = 128,
                              scale: float | None = None, o_part=None, lse_part=None, stream=None,
                              k_scale: float | None = None, v_scale: float | None = None):
    """Split-KV decode partials over a paged KV cache.

    q [B,Hq,d]; k_cache, v_cache: views [num_blocks, block_size, Hkv, d] with a
    contiguous last dimension (token-major pages as they are, head-major pages
    [num_blocks, Hkv, block_size, d] passed as ``.transpose(1, 2)``), both with
    the same strides; block_table [B, max_blocks] int32; seq_lens [B] int32.
    Returns (o_part [B,Hq,C,d], lse_part [B,Hq,C]) with
    C = ceil(max_blocks * block_size / chunk_size).  Caches of E4M3 codes
    (torch.float8_e4m3fn or uint8) take k_scale and v_scale (FP8 KV).
    """
    _check(q, "q")
    for t, n in ((k_cache, "k_cache"), (v_cache, "v_cache"), (block_table, "block_table"), (seq_lens, "seq_lens")):
        if not t.is_cuda:
            raise ValueError(f"{n} must be a GPU tensor")
    for t, n in ((k_cache, "k_cache"), (v_cache, "v_cache")):
        if t.dim() != 4 or t.stride(-1) != 1:
            raise ValueError(f"{n} must be a 4-D view with a contiguous last dimension")
    if k_cache.shape != v_cache.shape or k_cache.stride() != v_cache.stride():
        raise ValueError("k_cache and v_cache must have the same shape and strides")
    for t, n in ((block_table, "block_table"), (seq_lens, "seq_lens")):
        if t.dtype != torch.int32 or not t.is_contiguous():
            raise ValueError(f"{n} must be a contiguous int32 tensor")
    B, Hq, d = q.shape
    num_blocks, block_size, Hkv, dk = k_cache.shape
    max_blocks = block_table.shape[1]
    if dk != d or tuple(block_table.shape) != (B, max_blocks) or tuple(seq_lens.shape) != (B,):
        raise ValueError("shape mismatch between q, the caches, block_table and seq_lens")
    C = -(-(max_blocks * block_size) // chunk_size)
    if scale is None:
        scale = d ** -0.5
    if o_part is None:
        o_part = torch.empty((B, Hq, C, d), dtype=torch.float32, device=q.device)
    if lse_part is None:
        lse_part = torch.empty((B, Hq, C), dtype=torch.float32, device=q.device)
    pk = _lib.PagedKv(block_table.data_ptr(), seq_lens.data_ptr(), num_blocks, block_size, max_blocks,
                      k_cache.stride(0), k_cache.stride(1), k_cache.stride(2))
    if k_cache.dtype in (torch.uint8, torch.float8_e4m3fn):
        if k_scale is None or v_scale is None:
            raise ValueError("FP8 caches need k_scale and v_scale")
        st = _lib.load().attn_decode_paged_fp8kv_splitkv(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
                                                         float(k_scale), float(v_scale), ctypes.byref(pk),
                                                         o_part.data_ptr(), lse_part.data_ptr(), B, Hq, Hkv, d,
                                                         chunk_size, float(scale), _dtype_code(q), _stream(stream))
        if st != 0:
            raise AttnError(st, "attn_decode_paged_fp8kv_splitkv")
        return o_part, lse_part
    st = _lib.load().attn_decode_paged_splitkv(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
                                               ctypes.byref(pk), o_part.data_ptr(), lse_part.data_ptr(),
                                               B, Hq, Hkv, d, chunk_size, float(scale), _dtype_code(q),
                                               _stream(stream))
    if st != 0:
        raise AttnError(st, "attn_decode_paged_splitkv")
    return o_part, lse_part


def attn_decode_fp8kv_splitkv(q, k, v, k_scale: float, v_scale: float, chunk_size: int = 128,
                              scale: float | None = None, o_part=None, lse_part=None, stream=None):
    """q [B,Hq,d] fp16/bf16; k, v [B,Hkv,M,d] E4M3 codes (torch.float8_e4m3fn or uint8);
    K = k_scale * e4m3(k), V = v_scale * e4m3(v).  Returns (o_part, lse_part)."""
    _check(q, "q")
    for t, n in ((k, "k"), (v, "v")):
        _check(t, n)
        if t.dtype not in (torch.uint8, torch.float8_e4m3fn):
            raise TypeError(f"{n} must hold E4M3 codes (torch.float8_e4m3fn or uint8)")
    B, Hq, d = q.shape
    Hkv, M = k.shape[1], k.shape[2]
    C = -(-M // chunk_size)
    if scale is None:
        scale = d ** -0.5
    if o_part is None:
        o_part = torch.empty((B, Hq, C, d), dtype=torch.float32, device=q.device)
    if lse_part is None:
        lse_part = torch.empty((B, Hq, C), dtype=torch.float32, device=q.device)
    st = _lib.load().attn_decode_fp8kv_splitkv(q.data_ptr(), k.data_ptr(), v.data_ptr(), float(k_scale),
                                               float(v_scale), o_part.data_ptr(), lse_part.data_ptr(), B, Hq, Hkv,
                                               M, d, chunk_size, float(scale), _dtype_code(q), _stream(stream))
    if st != 0:
        raise AttnError(st, "attn_decode_fp8kv_splitkv")
    return o_part, lse_part


def attn_decode_fp8kv(q, k, v, k_scale: float, v_scale: float, chunk_size: int = 128,
                      scale: float | None = None, stream=None):
    """FP8-KV split-KV decode end to end (partials, then the merge)."""
    o_part, lse_part = attn_decode_fp8kv_splitkv(q, k, v, k_scale, v_scale, chunk_size, scale, stream=stream)
    o, lse = lse_merge(o_part, lse_part, q.dtype, stream=stream)
    return o, lse, o_part, lse_part


def attn_decode_paged(q, k_cache, v_cache, block_table, seq_lens, chunk_size: int = 128,
                      scale: float | None = None, stream=None, k_scale: float | None = None,
                      v_scale: float | None = None):
    """Paged split-KV decode end to end (partials, then the merge)."""
    o_part, lse_part = attn_decode_paged_splitkv(q, k_cache, v_cache, block_table, seq_lens, chunk_size,
                                                 scale, stream=stream, k_scale=k_scale, v_scale=v_scale)
    o, lse = lse_merge(o_part, lse_part, q.dtype, stream=stream)
    return o, lse, o_part, lse_part


def lse_merge(o_part, lse_part, out_dtype=torch.float16, o=None, lse=None, return_lse: bool = True,
              stream=None):
    """o_part [B,Hq,C,d], lse_part [B,Hq,C] -> (o [B,Hq,d] out_dtype, lse [B,Hq] fp32 or None)."""
    _check(o_part, "o_part")
    _check(lse_part, "lse_part")
    B, Hq, C, d = o_part.shape
    if o is None:
        o = torch.empty((B, Hq, d), dtype=out_dtype, device=o_part.device)
    if lse is None and return_lse:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=o_part.device)
    st = _lib.load().lse_merge(o_part.data_ptr(), lse_part.data_ptr(), o.data_ptr(),
                               lse.data_ptr() if lse is not None else None, B, Hq, C, d,
                               _DTYPES[o.dtype], _stream(stream))
    if st != 0:
        raise AttnError(st, "lse_merge")
    return o, lse


def attn_decode(q, k, v, chunk_size: int = 128, scale: float | None = None, stream=None):
    """Split-KV decode end to end (two launches on one stream)."""
    o_part, lse_part = attn_decode_splitkv(q, k, v, chunk_size, scale, stream=stream)
    o, lse = lse_merge(o_part, lse_part, q.dtype, stream=stream)
    return o, lse, o_part, lse_part
