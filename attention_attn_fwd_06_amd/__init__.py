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
    "AttnError", "ATTN_F16", "ATTN_BF16", "attn_fwd", "attn_fwd_fp8qk", "attn_decode_splitkv", "lse_merge",
    "attn_decode_workspace_bytes", "attn_status_string", "attn_decode", "attn_decode_paged_splitkv",
    "attn_decode_paged", "attn_decode_paged_fused", "attn_decode_fp8kv_splitkv", "attn_decode_fp8kv", "attn_decode_fused",
    "attn_decode_fused_workspace_bytes", "attn_decode_fused_noalloc", "attn_decode_fp8kv_fused",
]

ATTN_F16 = 0
ATTN_BF16 = 1
_FP8 = (torch.uint8, torch.float8_e4m3fn)
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


# Argument checks.  The C ABI receives bare pointers and sizes and cannot see a
# tensor's real extent, so every tensor is checked here against the shape,
# dtype and layout that the sizes passed to the library imply; a mismatch
# raises ValueError (TypeError for an unsupported dtype) before anything is
# launched.  Shapes and dtypes are checked first, the device last.

def _shape(t: torch.Tensor, name: str, shape):
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _dtype(t: torch.Tensor, name: str, dtype):
    if t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")


def _contig(t: torch.Tensor, name: str):
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _rows_contig(t: torch.Tensor, name: str, dim: int):
    if t.dim() != dim or t.stride(-1) != 1:
        raise ValueError(f"{name} must be {dim}-D with a contiguous last dimension")


def _devices(*named):
    """All given tensors (None entries skipped) on one GPU."""
    dev = None
    for t, name in named:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError(f"{name} is on {t.device}, the other tensors on {dev}")


def _check_f32(t, name, shape):
    _shape(t, name, shape)
    _dtype(t, name, torch.float32)
    _contig(t, name)


def _num_chunks(M: int, chunk_size: int) -> int:
    if int(chunk_size) <= 0:
        raise ValueError(f"chunk_size must be positive, got {chunk_size}")
    return -(-M // int(chunk_size))


def attn_fwd(q, k, v, causal: bool = False, scale: float | None = None, o=None, lse=None,
             return_lse: bool = True, stream=None):
    """q [B,N,Hq,d], k/v [B,M,Hkv,d] -> (o [B,N,Hq,d], lse [B,Hq,N] fp32 or None).

    q, k, v (and a given o) may be strided views (e.g. slices of a fused QKV
    projection, or head-major tensors transposed to [B,N,H,d]) as long as the
    last dimension is contiguous; they then go through attn_fwd_strided."""
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _rows_contig(t, n, 4)
    dt = _dtype_code(q)
    _dtype(k, "k", q.dtype)
    _dtype(v, "v", q.dtype)
    B, N, Hq, d = q.shape
    M, Hkv = k.shape[1], k.shape[2]
    _shape(k, "k", (B, M, Hkv, d))
    _shape(v, "v", k.shape)
    if o is not None:
        _rows_contig(o, "o", 4)
        _shape(o, "o", q.shape)
        _dtype(o, "o", q.dtype)
    if lse is not None:
        _check_f32(lse, "lse", (B, Hq, N))
    _devices((q, "q"), (k, "k"), (v, "v"), (o, "o"), (lse, "lse"))
    if scale is None:
        scale = d ** -0.5
    if o is None:
        o = torch.empty((B, N, Hq, d), dtype=q.dtype, device=q.device)
    if lse is None and return_lse:
        lse = torch.empty((B, Hq, N), dtype=torch.float32, device=q.device)
    lib = _lib.load()
    args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
            lse.data_ptr() if lse is not None else None,
            B, Hq, Hkv, N, M, d, int(bool(causal)), float(scale), dt)
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


def attn_fwd_fp8qk(q8, k8, v, q_scale: float, k_scale: float, causal: bool = False, scale: float | None = None,
                   o=None, lse=None, return_lse: bool = True, stream=None):
    """Prefill with Q and K as FP8 E4M3 codes (torch.float8_e4m3fn or uint8,
    contiguous) and per-tensor scales: Q = q_scale * e4m3(q8), K = k_scale *
    e4m3(k8).  q8 [B,N,Hq,d], k8 [B,M,Hkv,d], v [B,M,Hkv,d] fp16/bf16 ->
    (o [B,N,Hq,d] v.dtype, lse [B,Hq,N] fp32 or None)."""
    if q8.dim() != 4 or k8.dim() != 4 or v.dim() != 4:
        raise ValueError("q8, k8 and v must be 4-D")
    for t, n in ((q8, "q8"), (k8, "k8")):
        if t.dtype not in _FP8:
            raise TypeError(f"{n} must hold E4M3 codes (torch.float8_e4m3fn or uint8)")
    dt = _dtype_code(v)
    B, N, Hq, d = q8.shape
    M, Hkv = k8.shape[1], k8.shape[2]
    _shape(k8, "k8", (B, M, Hkv, d))
    _shape(v, "v", k8.shape)
    for t, n in ((q8, "q8"), (k8, "k8"), (v, "v")):
        _contig(t, n)
    if o is not None:
        _shape(o, "o", (B, N, Hq, d))
        _dtype(o, "o", v.dtype)
        _contig(o, "o")
    if lse is not None:
        _check_f32(lse, "lse", (B, Hq, N))
    _devices((q8, "q8"), (k8, "k8"), (v, "v"), (o, "o"), (lse, "lse"))
    if scale is None:
        scale = d ** -0.5
    if o is None:
        o = torch.empty((B, N, Hq, d), dtype=v.dtype, device=v.device)
    if lse is None and return_lse:
        lse = torch.empty((B, Hq, N), dtype=torch.float32, device=v.device)
    st = _lib.load().attn_fwd_fp8qk(q8.data_ptr(), k8.data_ptr(), v.data_ptr(), o.data_ptr(),
                                    lse.data_ptr() if lse is not None else None, float(q_scale), float(k_scale),
                                    B, Hq, Hkv, N, M, d, int(bool(causal)), float(scale), dt, _stream(stream))
    if st != 0:
        raise AttnError(st, "attn_fwd_fp8qk")
    return o, lse


def attn_decode_workspace_bytes(B: int, Hq: int, M: int, d: int, chunk_size: int = 128) -> int:
    return int(_lib.load().attn_decode_workspace_bytes(B, Hq, M, d, chunk_size))


def _decode_partials(q, o_part, lse_part, C):
    """Checks (or allocates) the fp32 partials of a split-KV decode of q."""
    B, Hq, d = q.shape
    if o_part is not None:
        _check_f32(o_part, "o_part", (B, Hq, C, d))
    if lse_part is not None:
        _check_f32(lse_part, "lse_part", (B, Hq, C))
    return o_part, lse_part


def _alloc_partials(q, o_part, lse_part, C):
    B, Hq, d = q.shape
    if o_part is None:
        o_part = torch.empty((B, Hq, C, d), dtype=torch.float32, device=q.device)
    if lse_part is None:
        lse_part = torch.empty((B, Hq, C), dtype=torch.float32, device=q.device)
    return o_part, lse_part


def attn_decode_splitkv(q, k, v, chunk_size: int = 128, scale: float | None = None,
                        o_part=None, lse_part=None, stream=None):
    """q [B,Hq,d], k/v [B,Hkv,M,d] -> (o_part [B,Hq,C,d] fp32, lse_part [B,Hq,C] fp32)."""
    if q.dim() != 3 or k.dim() != 4:
        raise ValueError("q must be [B, Hq, d] and k, v [B, Hkv, M, d]")
    dt = _dtype_code(q)
    B, Hq, d = q.shape
    Hkv, M = k.shape[1], k.shape[2]
    _shape(k, "k", (B, Hkv, M, d))
    _shape(v, "v", k.shape)
    _dtype(k, "k", q.dtype)
    _dtype(v, "v", q.dtype)
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _contig(t, n)
    C = _num_chunks(M, chunk_size)
    _decode_partials(q, o_part, lse_part, C)
    _devices((q, "q"), (k, "k"), (v, "v"), (o_part, "o_part"), (lse_part, "lse_part"))
    if scale is None:
        scale = d ** -0.5
    o_part, lse_part = _alloc_partials(q, o_part, lse_part, C)
    st = _lib.load().attn_decode_splitkv(q.data_ptr(), k.data_ptr(), v.data_ptr(), o_part.data_ptr(),
                                         lse_part.data_ptr(), B, Hq, Hkv, M, d, chunk_size,
                                         float(scale), dt, _stream(stream))
    if st != 0:
        raise AttnError(st, "attn_decode_splitkv")
    return o_part, lse_part


def attn_decode_fused_workspace_bytes(B: int, Hq: int, Hkv: int, M: int, d: int) -> int:
    return int(_lib.load().attn_decode_fused_workspace_bytes(B, Hq, Hkv, M, d))


def _fused_out_checks(q, o, lse, workspace, nbytes):
    """Checks of a fused decode's o [B,Hq,d] (q's dtype), lse [B,Hq] fp32 and
    uint8 workspace of at least nbytes, where given."""
    B, Hq, d = q.shape
    if o is not None:
        _shape(o, "o", (B, Hq, d))
        _dtype(o, "o", q.dtype)
        _contig(o, "o")
    if lse is not None:
        _check_f32(lse, "lse", (B, Hq))
    if workspace is not None:
        _dtype(workspace, "workspace", torch.uint8)
        _contig(workspace, "workspace")
        if workspace.numel() < nbytes:
            raise ValueError(f"workspace holds {workspace.numel()} bytes, {nbytes} needed")


def _fused_outputs(q, o, lse, return_lse, workspace, nbytes):
    """o, lse and workspace of a fused decode, allocated where not given (a
    fresh workspace is zero-filled)."""
    B, Hq, d = q.shape
    if o is None:
        o = torch.empty((B, Hq, d), dtype=q.dtype, device=q.device)
    if lse is None and return_lse:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    if workspace is None:
        workspace = torch.zeros(max(nbytes, 1), dtype=torch.uint8, device=q.device)
    return o, lse, workspace


def attn_decode_fused(q, k, v, scale: float | None = None, o=None, lse=None, return_lse: bool = True,
                      workspace=None, stream=None):
    """Split-KV decode end to end in one launch (partials and merge fused).

    q [B,Hq,d], k/v [B,Hkv,M,d] -> (o [B,Hq,d], lse [B,Hq] fp32 or None).
    ``workspace``: a uint8 GPU tensor of at least
    attn_decode_fused_workspace_bytes(B, Hq, Hkv, M, d) bytes, zero-filled
    before its first use (every completed call leaves its counters at zero);
    by default a fresh zeroed one is allocated for the call."""
    if q.dim() != 3 or k.dim() != 4:
        raise ValueError("q must be [B, Hq, d] and k, v [B, Hkv, M, d]")
    dt = _dtype_code(q)
    B, Hq, d = q.shape
    Hkv, M = k.shape[1], k.shape[2]
    _shape(k, "k", (B, Hkv, M, d))
    _shape(v, "v", k.shape)
    _dtype(k, "k", q.dtype)
    _dtype(v, "v", q.dtype)
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _contig(t, n)
    nbytes = attn_decode_fused_workspace_bytes(B, Hq, Hkv, M, d)
    _fused_out_checks(q, o, lse, workspace, nbytes)
    _devices((q, "q"), (k, "k"), (v, "v"), (o, "o"), (lse, "lse"), (workspace, "workspace"))
    if scale is None:
        scale = d ** -0.5
    o, lse, workspace = _fused_outputs(q, o, lse, return_lse, workspace, nbytes)
    st = _lib.load().attn_decode_fused(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                       lse.data_ptr() if lse is not None else None, workspace.data_ptr(),
                                       workspace.numel(), B, Hq, Hkv, M, d, float(scale), dt, _stream(stream))
    if st != 0:
        raise AttnError(st, "attn_decode_fused")
    return o, lse


def attn_decode_fused_noalloc(q, k, v, scale: float | None = None, o=None, lse=None, return_lse: bool = True,
                              stream=None):
    """attn_decode_fused on the library's static scratch (no workspace, no
    device allocation by the library; o and lse are allocated here unless
    given).  Calls that overlap on one GPU race."""
    if q.dim() != 3 or k.dim() != 4:
        raise ValueError("q must be [B, Hq, d] and k, v [B, Hkv, M, d]")
    dt = _dtype_code(q)
    B, Hq, d = q.shape
    Hkv, M = k.shape[1], k.shape[2]
    _shape(k, "k", (B, Hkv, M, d))
    _shape(v, "v", k.shape)
    _dtype(k, "k", q.dtype)
    _dtype(v, "v", q.dtype)
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _contig(t, n)
    _fused_out_checks(q, o, lse, None, 0)
    _devices((q, "q"), (k, "k"), (v, "v"), (o, "o"), (lse, "lse"))
    if scale is None:
        scale = d ** -0.5
    if o is None:
        o = torch.empty((B, Hq, d), dtype=q.dtype, device=q.device)
    if lse is None and return_lse:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    st = _lib.load().attn_decode_fused_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                               lse.data_ptr() if lse is not None else None, B, Hq, Hkv, M, d,
                                               float(scale), dt, _stream(stream))
    if st != 0:
        raise AttnError(st, "attn_decode_fused_noalloc")
    return o, lse


def _paged_args(q, k_cache, v_cache, block_table, seq_lens):
    """Checks of a paged call's inputs; returns (dtype code, B, Hq, d,
    num_blocks, block_size, Hkv, max_blocks)."""
    if q.dim() != 3:
        raise ValueError("q must be [B, Hq, d]")
    dt = _dtype_code(q)
    _contig(q, "q")
    for t, n in ((k_cache, "k_cache"), (v_cache, "v_cache")):
        _rows_contig(t, n, 4)
    if k_cache.shape != v_cache.shape or k_cache.stride() != v_cache.stride():
        raise ValueError("k_cache and v_cache must have the same shape and strides")
    if k_cache.dtype in _FP8:
        if v_cache.dtype not in _FP8:
            raise ValueError("k_cache holds E4M3 codes, so v_cache must too")
    else:
        _dtype(k_cache, "k_cache", q.dtype)
        _dtype(v_cache, "v_cache", q.dtype)
    for t, n in ((block_table, "block_table"), (seq_lens, "seq_lens")):
        if t.dtype != torch.int32 or not t.is_contiguous():
            raise ValueError(f"{n} must be a contiguous int32 tensor")
    B, Hq, d = q.shape
    num_blocks, block_size, Hkv, dk = k_cache.shape
    if block_table.dim() != 2:
        raise ValueError("block_table must be [B, max_blocks]")
    max_blocks = block_table.shape[1]
    if dk != d or tuple(block_table.shape) != (B, max_blocks) or tuple(seq_lens.shape) != (B,):
        raise ValueError("shape mismatch between q, the caches, block_table and seq_lens")
    return dt, B, Hq, d, num_blocks, block_size, Hkv, max_blocks


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
    fp8 = k_cache.dtype in _FP8
    if fp8 and (k_scale is None or v_scale is None):
        raise ValueError("FP8 caches need k_scale and v_scale")
    dt, B, Hq, d, num_blocks, block_size, Hkv, max_blocks = _paged_args(q, k_cache, v_cache, block_table, seq_lens)
    C = _num_chunks(max_blocks * block_size, chunk_size)
    _decode_partials(q, o_part, lse_part, C)
    _devices((q, "q"), (k_cache, "k_cache"), (v_cache, "v_cache"), (block_table, "block_table"),
             (seq_lens, "seq_lens"), (o_part, "o_part"), (lse_part, "lse_part"))
    if scale is None:
        scale = d ** -0.5
    o_part, lse_part = _alloc_partials(q, o_part, lse_part, C)
    pk = _lib.PagedKv(block_table.data_ptr(), seq_lens.data_ptr(), num_blocks, block_size, max_blocks,
                      k_cache.stride(0), k_cache.stride(1), k_cache.stride(2))
    if fp8:
        st = _lib.load().attn_decode_paged_fp8kv_splitkv(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
                                                         float(k_scale), float(v_scale), ctypes.byref(pk),
                                                         o_part.data_ptr(), lse_part.data_ptr(), B, Hq, Hkv, d,
                                                         chunk_size, float(scale), dt, _stream(stream))
        if st != 0:
            raise AttnError(st, "attn_decode_paged_fp8kv_splitkv")
        return o_part, lse_part
    st = _lib.load().attn_decode_paged_splitkv(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
                                               ctypes.byref(pk), o_part.data_ptr(), lse_part.data_ptr(),
                                               B, Hq, Hkv, d, chunk_size, float(scale), dt, _stream(stream))
    if st != 0:
        raise AttnError(st, "attn_decode_paged_splitkv")
    return o_part, lse_part


def attn_decode_paged_fused(q, k_cache, v_cache, block_table, seq_lens, scale: float | None = None, o=None,
                            lse=None, return_lse: bool = True, workspace=None, stream=None,
                            k_scale: float | None = None, v_scale: float | None = None):
    """Split-KV decode over a paged KV cache in one launch (partials of
    128-key chunk runs and their merge fused).

    q [B,Hq,d]; k_cache, v_cache, block_table, seq_lens as in
    attn_decode_paged_splitkv.  Returns (o [B,Hq,d], lse [B,Hq] fp32 or
    None).  Caches of E4M3 codes (torch.float8_e4m3fn or uint8) take k_scale
    and v_scale (attn_decode_paged_fp8kv_fused).  ``workspace``: a uint8 GPU
    tensor of at least attn_decode_fused_workspace_bytes(B, Hq, Hkv,
    max_blocks * block_size, d) bytes, zero-filled before its first use; by
    default a fresh zeroed one."""
    fp8 = k_cache.dtype in _FP8
    if fp8 and (k_scale is None or v_scale is None):
        raise ValueError("FP8 caches need k_scale and v_scale")
    dt, B, Hq, d, num_blocks, block_size, Hkv, max_blocks = _paged_args(q, k_cache, v_cache, block_table, seq_lens)
    nbytes = attn_decode_fused_workspace_bytes(B, Hq, Hkv, max_blocks * block_size, d)
    _fused_out_checks(q, o, lse, workspace, nbytes)
    _devices((q, "q"), (k_cache, "k_cache"), (v_cache, "v_cache"), (block_table, "block_table"),
             (seq_lens, "seq_lens"), (o, "o"), (lse, "lse"), (workspace, "workspace"))
    if scale is None:
        scale = d ** -0.5
    o, lse, workspace = _fused_outputs(q, o, lse, return_lse, workspace, nbytes)
    pk = _lib.PagedKv(block_table.data_ptr(), seq_lens.data_ptr(), num_blocks, block_size, max_blocks,
                      k_cache.stride(0), k_cache.stride(1), k_cache.stride(2))
    lse_ptr = lse.data_ptr() if lse is not None else None
    if fp8:
        st = _lib.load().attn_decode_paged_fp8kv_fused(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
                                                       float(k_scale), float(v_scale), ctypes.byref(pk), o.data_ptr(),
                                                       lse_ptr, workspace.data_ptr(), workspace.numel(), B, Hq, Hkv,
                                                       d, float(scale), dt, _stream(stream))
        if st != 0:
            raise AttnError(st, "attn_decode_paged_fp8kv_fused")
        return o, lse
    st = _lib.load().attn_decode_paged_fused(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), ctypes.byref(pk),
                                             o.data_ptr(), lse_ptr, workspace.data_ptr(), workspace.numel(), B, Hq,
                                             Hkv, d, float(scale), dt, _stream(stream))
    if st != 0:
        raise AttnError(st, "attn_decode_paged_fused")
    return o, lse


def attn_decode_fp8kv_splitkv(q, k, v, k_scale: float, v_scale: float, chunk_size: int = 128,
                              scale: float | None = None, o_part=None, lse_part=None, stream=None):
    """q [B,Hq,d] fp16/bf16; k, v [B,Hkv,M,d] E4M3 codes (torch.float8_e4m3fn or uint8);
    K = k_scale * e4m3(k), V = v_scale * e4m3(v).  Returns (o_part, lse_part)."""
    if q.dim() != 3 or k.dim() != 4:
        raise ValueError("q must be [B, Hq, d] and k, v [B, Hkv, M, d]")
    dt = _dtype_code(q)
    for t, n in ((k, "k"), (v, "v")):
        if t.dtype not in _FP8:
            raise TypeError(f"{n} must hold E4M3 codes (torch.float8_e4m3fn or uint8)")
    B, Hq, d = q.shape
    Hkv, M = k.shape[1], k.shape[2]
    _shape(k, "k", (B, Hkv, M, d))
    _shape(v, "v", k.shape)
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _contig(t, n)
    C = _num_chunks(M, chunk_size)
    _decode_partials(q, o_part, lse_part, C)
    _devices((q, "q"), (k, "k"), (v, "v"), (o_part, "o_part"), (lse_part, "lse_part"))
    if scale is None:
        scale = d ** -0.5
    o_part, lse_part = _alloc_partials(q, o_part, lse_part, C)
    st = _lib.load().attn_decode_fp8kv_splitkv(q.data_ptr(), k.data_ptr(), v.data_ptr(), float(k_scale),
                                               float(v_scale), o_part.data_ptr(), lse_part.data_ptr(), B, Hq, Hkv,
                                               M, d, chunk_size, float(scale), dt, _stream(stream))
    if st != 0:
        raise AttnError(st, "attn_decode_fp8kv_splitkv")
    return o_part, lse_part


def attn_decode_fp8kv_fused(q, k, v, k_scale: float, v_scale: float, scale: float | None = None, o=None,
                            lse=None, return_lse: bool = True, workspace=None, stream=None):
    """FP8-KV split-KV decode end to end in one launch (partials and merge
    fused).  q [B,Hq,d] fp16/bf16; k, v [B,Hkv,M,d] E4M3 codes
    (torch.float8_e4m3fn or uint8); K = k_scale * e4m3(k), V = v_scale *
    e4m3(v).  Returns (o [B,Hq,d] q.dtype, lse [B,Hq] fp32 or None);
    ``workspace`` as in attn_decode_fused."""
    if q.dim() != 3 or k.dim() != 4:
        raise ValueError("q must be [B, Hq, d] and k, v [B, Hkv, M, d]")
    dt = _dtype_code(q)
    for t, n in ((k, "k"), (v, "v")):
        if t.dtype not in _FP8:
            raise TypeError(f"{n} must hold E4M3 codes (torch.float8_e4m3fn or uint8)")
    B, Hq, d = q.shape
    Hkv, M = k.shape[1], k.shape[2]
    _shape(k, "k", (B, Hkv, M, d))
    _shape(v, "v", k.shape)
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _contig(t, n)
    nbytes = attn_decode_fused_workspace_bytes(B, Hq, Hkv, M, d)
    _fused_out_checks(q, o, lse, workspace, nbytes)
    _devices((q, "q"), (k, "k"), (v, "v"), (o, "o"), (lse, "lse"), (workspace, "workspace"))
    if scale is None:
        scale = d ** -0.5
    o, lse, workspace = _fused_outputs(q, o, lse, return_lse, workspace, nbytes)
    st = _lib.load().attn_decode_fp8kv_fused(q.data_ptr(), k.data_ptr(), v.data_ptr(), float(k_scale),
                                             float(v_scale), o.data_ptr(), lse.data_ptr() if lse is not None else None,
                                             workspace.data_ptr(), workspace.numel(), B, Hq, Hkv, M, d, float(scale),
                                             dt, _stream(stream))
    if st != 0:
        raise AttnError(st, "attn_decode_fp8kv_fused")
    return o, lse


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
    if o_part.dim() != 4:
        raise ValueError("o_part must be [B, Hq, C, d]")
    B, Hq, C, d = o_part.shape
    _check_f32(o_part, "o_part", (B, Hq, C, d))
    _check_f32(lse_part, "lse_part", (B, Hq, C))
    if o is not None:
        _dtype_code(o)
        _shape(o, "o", (B, Hq, d))
        _contig(o, "o")
    else:
        if out_dtype not in _DTYPES:
            raise TypeError(f"unsupported dtype {out_dtype}; expected float16 or bfloat16")
    if lse is not None:
        _check_f32(lse, "lse", (B, Hq))
    _devices((o_part, "o_part"), (lse_part, "lse_part"), (o, "o"), (lse, "lse"))
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
