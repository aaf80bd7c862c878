"""The C ABI without a GPU: the library loads, exports every function that
include/attn.h declares, and rejects every invalid argument with its
documented status before touching the GPU.  No call here has a complete set
of valid arguments, so nothing is ever launched."""
import ctypes
import pathlib
import re

import pytest

from attention_attn_fwd_06_amd import _lib

HEADER = pathlib.Path(__file__).resolve().parents[1] / "include" / "attn.h"
FAKE = 4096  # a 16-byte-aligned non-null address; never dereferenced


def declared_functions():
    text = re.sub(r"/\*.*?\*/", "", HEADER.read_text(), flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\*?(\w+)\s*\(", text, flags=re.M)))


def status_codes():
    text = HEADER.read_text()
    return {m.group(1): int(m.group(2)) for m in re.finditer(r"(ATTN_\w+)\s*=\s*(-?\d+)", text)}


def test_header_declares_expected_api():
    assert declared_functions() == sorted(
        ["attn_fwd", "attn_fwd_strided", "attn_decode_workspace_bytes", "attn_decode_splitkv",
         "attn_decode_paged_splitkv", "attn_decode_paged_fp8kv_splitkv", "attn_decode_fp8kv_splitkv", "lse_merge",
         "attn_status_string", "attn_decode_fused_workspace_bytes", "attn_decode_fused",
         "attn_decode_fused_noalloc", "attn_fwd_fp8qk", "attn_decode_paged_fused", "attn_decode_fp8kv_fused",
         "attn_decode_paged_fp8kv_fused"])


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(str(_lib.LIB_PATH))
    for name in declared_functions():
        assert hasattr(lib, name), name
    assert set(declared_functions()) == set(_lib.SYMBOLS)


def test_status_strings():
    lib = _lib.load()
    codes = status_codes()
    seen = set()
    for name, val in codes.items():
        if name in ("ATTN_F16", "ATTN_BF16"):
            continue
        s = lib.attn_status_string(val).decode()
        assert s and s != "unknown status", name
        seen.add(s)
    assert len(seen) == len([n for n in codes if n not in ("ATTN_F16", "ATTN_BF16")])
    assert lib.attn_status_string(12345).decode() == "unknown status"


def fwd(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=None, B=1, Hq=2, Hkv=2, N=128, M=128, d=64,
             causal=0, scale=0.125, dtype=0, stream=None)
    a.update(kw)
    return _lib.load().attn_fwd(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["Hq"], a["Hkv"],
                                a["N"], a["M"], a["d"], a["causal"], a["scale"], a["dtype"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), -1), (dict(k=None), -1), (dict(v=None), -1), (dict(o=None), -1),
    (dict(B=0), -2), (dict(Hq=-1), -2), (dict(Hkv=0), -2), (dict(N=0), -2), (dict(M=-5), -2), (dict(d=0), -2),
    (dict(d=96), -3), (dict(d=512), -3), (dict(d=16), -3),
    (dict(dtype=2), -4), (dict(dtype=-1), -4),
    (dict(Hq=6, Hkv=4), -5),
    (dict(causal=1, N=256, M=128), -6),
    (dict(scale=-0.5), -11), (dict(scale=float("inf")), -11), (dict(scale=float("nan")), -11),
    (dict(B=1 << 14, Hq=1 << 12, Hkv=1, N=1 << 12), -9),   # grid of 2^32 workgroups
    (dict(M=1 << 23, Hkv=2, d=128), -9),                 # one batch's K beyond 2^31 elements
    (dict(q=FAKE + 8), -10), (dict(o=FAKE + 2), -10), (dict(lse=FAKE + 2), -10),
])
def test_attn_fwd_rejects(kw, code):
    assert fwd(**kw) == code


def contiguous_strides(B=1, Hq=2, Hkv=2, N=128, M=128, d=64):
    s = _lib.Strides()
    s.q[:] = [N * Hq * d, Hq * d, d]
    s.o[:] = [N * Hq * d, Hq * d, d]
    s.k[:] = [M * Hkv * d, Hkv * d, d]
    s.v[:] = [M * Hkv * d, Hkv * d, d]
    return s


def fwd_strided(edit=None, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=None, B=1, Hq=2, Hkv=2, N=128, M=128, d=64,
             causal=0, scale=0.125, dtype=0, stream=None)
    a.update(kw)
    st = contiguous_strides(a["B"], a["Hq"], a["Hkv"], a["N"], a["M"], a["d"])
    if edit:
        edit(st)
    return _lib.load().attn_fwd_strided(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["Hq"],
                                        a["Hkv"], a["N"], a["M"], a["d"], a["causal"], a["scale"],
                                        a["dtype"], ctypes.byref(st), a["stream"])


def _set(field, i, val):
    def edit(st):
        getattr(st, field)[i] = val
    return edit


@pytest.mark.parametrize("edit,kw,code", [
    (None, dict(q=None), -1), (None, dict(N=0), -2), (None, dict(d=96), -3), (None, dict(dtype=3), -4),
    (None, dict(Hq=6, Hkv=4), -5), (None, dict(causal=1, N=256, M=128), -6),
    (None, dict(scale=float("nan")), -11),
    (_set("q", 1, -128), {}, -12), (_set("o", 2, 4), {}, -12), (_set("v", 0, 12), {}, -12),
    (_set("v", 1, 256), {}, -12),      # k and v token strides differ
    (_set("k", 1, 32), {}, -12),       # token stride below d (same for v)
    (None, dict(q=FAKE + 8), -10),
])
def test_attn_fwd_strided_rejects(edit, kw, code):
    assert fwd_strided(edit, **kw) == code


def test_attn_fwd_strided_kv_slice_too_large():
    """(M + 64) token rows of the k/v token stride beyond 2^31 elements."""
    def edit(st):
        st.k[1] = 1 << 24
        st.v[1] = 1 << 24
    assert fwd_strided(edit) == -9


def test_attn_fwd_strided_k_v_equal_small_token_stride_rejected():
    def edit(st):
        st.k[1] = 32
        st.v[1] = 32
    assert fwd_strided(edit) == -12


def dec(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, op=FAKE, lp=FAKE, B=1, Hq=8, Hkv=8, M=512, d=128, chunk=128,
             scale=0.088, dtype=0, stream=None)
    a.update(kw)
    return _lib.load().attn_decode_splitkv(a["q"], a["k"], a["v"], a["op"], a["lp"], a["B"], a["Hq"],
                                           a["Hkv"], a["M"], a["d"], a["chunk"], a["scale"], a["dtype"],
                                           a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), -1), (dict(op=None), -1), (dict(lp=None), -1),
    (dict(M=0), -2), (dict(chunk=0), -2), (dict(B=-1), -2),
    (dict(d=80), -3), (dict(d=512), -3), (dict(dtype=7), -4), (dict(Hq=8, Hkv=3), -5),
    (dict(chunk=64), -7), (dict(chunk=192), -7), (dict(chunk=8320), -7),
    (dict(scale=-1.0), -11),
    (dict(B=70000, Hq=1, Hkv=1, M=128), -9),
    (dict(k=FAKE + 4), -10), (dict(op=FAKE + 1), -10),
])
def test_decode_rejects(kw, code):
    assert dec(**kw) == code


def paged(**kw):
    """attn_decode_paged_splitkv with a page table whose pointers are fake."""
    a = dict(q=FAKE, kc=FAKE, vc=FAKE, op=FAKE, lp=FAKE, B=2, Hq=8, Hkv=2, d=128, chunk=128, scale=0.088,
             dtype=1, stream=None, bt=FAKE, sl=FAKE, nb=64, bs=16, mb=32, ps=16 * 2 * 128, ts=2 * 128, hs=128,
             pages=True)
    a.update(kw)
    pk = _lib.PagedKv(a["bt"], a["sl"], a["nb"], a["bs"], a["mb"], a["ps"], a["ts"], a["hs"])
    return _lib.load().attn_decode_paged_splitkv(a["q"], a["kc"], a["vc"], ctypes.byref(pk) if a["pages"] else None,
                                                 a["op"], a["lp"], a["B"], a["Hq"], a["Hkv"], a["d"], a["chunk"],
                                                 a["scale"], a["dtype"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), -1), (dict(kc=None), -1), (dict(pages=False), -1), (dict(bt=None), -1), (dict(sl=None), -1),
    (dict(op=None), -1),
    (dict(B=0), -2), (dict(nb=0), -2), (dict(bs=0), -2), (dict(mb=0), -2),
    (dict(d=96), -3), (dict(dtype=2), -4), (dict(Hq=8, Hkv=3), -5), (dict(chunk=100), -7),
    (dict(scale=float("nan")), -11),
    (dict(bs=24), -12), (dict(ts=-8), -12), (dict(ps=12), -12), (dict(hs=4), -12), (dict(ts=1 << 28), -12),
    (dict(mb=1 << 26, bs=16), -9), (dict(B=70000, Hq=1, Hkv=1), -9),
    (dict(kc=FAKE + 8), -10), (dict(bt=FAKE + 2), -10), (dict(lp=FAKE + 2), -10),
])
def test_paged_decode_rejects(kw, code):
    assert paged(**kw) == code


def fp8(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, ks=0.01, vs=2.0, op=FAKE, lp=FAKE, B=1, Hq=8, Hkv=2, M=512, d=128, chunk=128,
             scale=0.088, dtype=1, stream=None)
    a.update(kw)
    return _lib.load().attn_decode_fp8kv_splitkv(a["q"], a["k"], a["v"], a["ks"], a["vs"], a["op"], a["lp"], a["B"],
                                                 a["Hq"], a["Hkv"], a["M"], a["d"], a["chunk"], a["scale"],
                                                 a["dtype"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(k=None), -1), (dict(lp=None), -1), (dict(M=0), -2), (dict(d=48), -3), (dict(d=256), -3),
    (dict(dtype=5), -4),
    (dict(Hq=6, Hkv=4), -5), (dict(chunk=96), -7), (dict(ks=-1.0), -11), (dict(vs=float("inf")), -11),
    (dict(ks=float("nan")), -11), (dict(B=70000, Hq=1, Hkv=1), -9), (dict(v=FAKE + 8), -10),
])
def test_fp8kv_decode_rejects(kw, code):
    assert fp8(**kw) == code


def paged8(**kw):
    a = dict(q=FAKE, kc=FAKE, vc=FAKE, ks=0.01, vs=0.02, op=FAKE, lp=FAKE, B=2, Hq=8, Hkv=2, d=128, chunk=128,
             scale=0.088, dtype=1, stream=None, bt=FAKE, sl=FAKE, nb=64, bs=16, mb=32, ps=16 * 2 * 128, ts=2 * 128,
             hs=128)
    a.update(kw)
    pk = _lib.PagedKv(a["bt"], a["sl"], a["nb"], a["bs"], a["mb"], a["ps"], a["ts"], a["hs"])
    return _lib.load().attn_decode_paged_fp8kv_splitkv(a["q"], a["kc"], a["vc"], a["ks"], a["vs"], ctypes.byref(pk),
                                                       a["op"], a["lp"], a["B"], a["Hq"], a["Hkv"], a["d"],
                                                       a["chunk"], a["scale"], a["dtype"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(kc=None), -1), (dict(bt=None), -1), (dict(mb=0), -2), (dict(d=80), -3), (dict(d=256), -3),
    (dict(chunk=64), -7), (dict(ks=-0.5), -11), (dict(vs=float("nan")), -11),
    (dict(hs=8), -12), (dict(ts=24), -12), (dict(bs=8), -12), (dict(vc=FAKE + 8), -10),
])
def test_paged_fp8kv_decode_rejects(kw, code):
    assert paged8(**kw) == code


def mrg(**kw):
    a = dict(op=FAKE, lp=FAKE, o=FAKE, lse=None, B=1, Hq=8, C=4, d=128, dtype=0, stream=None)
    a.update(kw)
    return _lib.load().lse_merge(a["op"], a["lp"], a["o"], a["lse"], a["B"], a["Hq"], a["C"], a["d"],
                                 a["dtype"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(op=None), -1), (dict(o=None), -1), (dict(C=0), -2), (dict(d=100), -3), (dict(dtype=3), -4),
    (dict(o=FAKE + 1), -10), (dict(lse=FAKE + 1), -10), (dict(op=FAKE + 4), -10),
])
def test_merge_rejects(kw, code):
    assert mrg(**kw) == code


def test_workspace_bytes():
    lib = _lib.load()
    assert lib.attn_decode_workspace_bytes(2, 8, 65536, 128, 128) == 2 * 8 * 512 * 129 * 4
    assert lib.attn_decode_workspace_bytes(1, 8, 513, 128, 128) == 1 * 8 * 5 * 129 * 4
    assert lib.attn_decode_workspace_bytes(0, 8, 512, 128, 128) == 0
    # head dim 256 (16-bit decode, fused decode, merge)
    assert lib.attn_decode_workspace_bytes(1, 4, 300, 256, 128) == 1 * 4 * 3 * 257 * 4
    assert lib.attn_decode_fused_workspace_bytes(2, 16, 4, 1000, 256) > 0


def fused(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=None, ws=FAKE, wsb=1 << 30, B=2, Hq=8, Hkv=8, M=65536, d=128,
             scale=0.088, dtype=0, stream=None)
    a.update(kw)
    return _lib.load().attn_decode_fused(a["q"], a["k"], a["v"], a["o"], a["lse"], a["ws"], a["wsb"], a["B"],
                                         a["Hq"], a["Hkv"], a["M"], a["d"], a["scale"], a["dtype"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), -1), (dict(o=None), -1), (dict(M=0), -2), (dict(Hkv=0), -2), (dict(d=80), -3),
    (dict(dtype=3), -4), (dict(Hq=8, Hkv=3), -5), (dict(scale=float("nan")), -11),
    (dict(B=70000, Hq=1, Hkv=1), -9), (dict(M=1 << 24), -9),
    (dict(o=FAKE + 8), -10), (dict(lse=FAKE + 1), -10),
    (dict(ws=None), -13), (dict(ws=FAKE + 8), -13), (dict(wsb=100), -13),
])
def test_decode_fused_rejects(kw, code):
    assert fused(**kw) == code


def test_decode_fused_workspace_bytes():
    lib = _lib.load()
    # long decode workload: 16 rows of 512 chunks; at most 256 segments each,
    # one fp32 output row of 128 and one lse per segment, plus the counters
    n = lib.attn_decode_fused_workspace_bytes(2, 8, 8, 65536, 128)
    assert n == 256 + 16 * 256 * 4 + 16 * 256 * 128 * 4
    assert fused(wsb=n - 1) == -13
    assert lib.attn_decode_fused_workspace_bytes(2, 8, 3, 100, 128) == 0
    assert lib.attn_decode_fused_workspace_bytes(2, 8, 8, 100, 96) == 0


def pfused(**kw):
    """attn_decode_paged_fused with a page table whose pointers are fake."""
    a = dict(q=FAKE, kc=FAKE, vc=FAKE, o=FAKE, lse=None, ws=FAKE, wsb=1 << 30, B=2, Hq=8, Hkv=2, d=128, scale=0.088,
             dtype=1, stream=None, bt=FAKE, sl=FAKE, nb=64, bs=16, mb=32, ps=16 * 2 * 128, ts=2 * 128, hs=128,
             pages=True)
    a.update(kw)
    pk = _lib.PagedKv(a["bt"], a["sl"], a["nb"], a["bs"], a["mb"], a["ps"], a["ts"], a["hs"])
    return _lib.load().attn_decode_paged_fused(a["q"], a["kc"], a["vc"], ctypes.byref(pk) if a["pages"] else None,
                                               a["o"], a["lse"], a["ws"], a["wsb"], a["B"], a["Hq"], a["Hkv"], a["d"],
                                               a["scale"], a["dtype"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), -1), (dict(o=None), -1), (dict(pages=False), -1), (dict(sl=None), -1),
    (dict(B=0), -2), (dict(bs=0), -2), (dict(d=80), -3), (dict(dtype=2), -4), (dict(Hq=8, Hkv=3), -5),
    (dict(scale=-1.0), -11), (dict(bs=24), -12), (dict(ts=-8), -12),
    (dict(o=FAKE + 8), -10), (dict(lse=FAKE + 1), -10), (dict(vc=FAKE + 8), -10),
    (dict(ws=None), -13), (dict(ws=FAKE + 8), -13), (dict(wsb=100), -13),
])
def test_decode_paged_fused_rejects(kw, code):
    assert pfused(**kw) == code


def test_decode_paged_fused_workspace_is_that_of_the_longest_sequence():
    lib = _lib.load()
    n = lib.attn_decode_fused_workspace_bytes(2, 8, 2, 32 * 16, 128)
    assert n > 0 and pfused(wsb=n - 1) == -13


def fused8(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, ks=0.01, vs=2.0, o=FAKE, lse=None, ws=FAKE, wsb=1 << 30, B=1, Hq=8, Hkv=2,
             M=512, d=128, scale=0.088, dtype=1, stream=None)
    a.update(kw)
    return _lib.load().attn_decode_fp8kv_fused(a["q"], a["k"], a["v"], a["ks"], a["vs"], a["o"], a["lse"], a["ws"],
                                               a["wsb"], a["B"], a["Hq"], a["Hkv"], a["M"], a["d"], a["scale"],
                                               a["dtype"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(k=None), -1), (dict(o=None), -1), (dict(M=0), -2), (dict(d=48), -3), (dict(d=256), -3),
    (dict(dtype=5), -4), (dict(Hq=6, Hkv=4), -5), (dict(ks=-1.0), -11), (dict(vs=float("inf")), -11),
    (dict(scale=float("nan")), -11), (dict(B=70000, Hq=1, Hkv=1), -9), (dict(v=FAKE + 8), -10),
    (dict(o=FAKE + 8), -10), (dict(lse=FAKE + 1), -10),
    (dict(ws=None), -13), (dict(ws=FAKE + 8), -13), (dict(wsb=100), -13),
])
def test_fp8kv_decode_fused_rejects(kw, code):
    assert fused8(**kw) == code


def pfused8(**kw):
    """attn_decode_paged_fp8kv_fused with a page table whose pointers are fake."""
    a = dict(q=FAKE, kc=FAKE, vc=FAKE, ks=0.01, vs=0.02, o=FAKE, lse=None, ws=FAKE, wsb=1 << 30, B=2, Hq=8, Hkv=2,
             d=128, scale=0.088, dtype=1, stream=None, bt=FAKE, sl=FAKE, nb=64, bs=16, mb=32, ps=16 * 2 * 128,
             ts=2 * 128, hs=128)
    a.update(kw)
    pk = _lib.PagedKv(a["bt"], a["sl"], a["nb"], a["bs"], a["mb"], a["ps"], a["ts"], a["hs"])
    return _lib.load().attn_decode_paged_fp8kv_fused(a["q"], a["kc"], a["vc"], a["ks"], a["vs"], ctypes.byref(pk),
                                                     a["o"], a["lse"], a["ws"], a["wsb"], a["B"], a["Hq"], a["Hkv"],
                                                     a["d"], a["scale"], a["dtype"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(kc=None), -1), (dict(o=None), -1), (dict(bt=None), -1), (dict(mb=0), -2), (dict(d=80), -3),
    (dict(d=256), -3), (dict(dtype=2), -4), (dict(ks=-0.5), -11), (dict(vs=float("nan")), -11),
    (dict(hs=8), -12), (dict(ts=24), -12), (dict(bs=8), -12), (dict(vc=FAKE + 8), -10), (dict(o=FAKE + 8), -10),
    (dict(ws=None), -13), (dict(ws=FAKE + 8), -13), (dict(wsb=100), -13),
])
def test_paged_fp8kv_decode_fused_rejects(kw, code):
    assert pfused8(**kw) == code


def noalloc(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=None, B=2, Hq=8, Hkv=8, M=65536, d=128, scale=0.088, dtype=0,
             stream=None)
    a.update(kw)
    return _lib.load().attn_decode_fused_noalloc(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["Hq"], a["Hkv"],
                                                 a["M"], a["d"], a["scale"], a["dtype"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), -1), (dict(o=None), -1), (dict(M=0), -2), (dict(d=80), -3), (dict(dtype=3), -4),
    (dict(Hq=8, Hkv=3), -5), (dict(scale=-1.0), -11), (dict(B=70000, Hq=1, Hkv=1), -9), (dict(o=FAKE + 8), -10),
    # 64 rows of 16 heads, 512 chunks: 64 segments each need 33.8 MB of partials
    (dict(B=64, Hq=16, Hkv=1), -14),
])
def test_decode_fused_noalloc_rejects(kw, code):
    assert noalloc(**kw) == code


def fp8qk(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=None, qs=0.01, ks=0.02, B=1, Hq=4, Hkv=2, N=128, M=128, d=128,
             causal=1, scale=0.088, dtype=1, stream=None)
    a.update(kw)
    return _lib.load().attn_fwd_fp8qk(a["q"], a["k"], a["v"], a["o"], a["lse"], a["qs"], a["ks"], a["B"], a["Hq"],
                                      a["Hkv"], a["N"], a["M"], a["d"], a["causal"], a["scale"], a["dtype"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), -1), (dict(v=None), -1), (dict(N=0), -2), (dict(d=32), -3), (dict(d=256), -3), (dict(dtype=4), -4),
    (dict(Hq=6, Hkv=4), -5), (dict(causal=1, N=256, M=128), -6), (dict(qs=-1.0), -11), (dict(ks=float("nan")), -11),
    (dict(scale=float("inf")), -11), (dict(M=1 << 23, Hkv=2), -9), (dict(k=FAKE + 8), -10), (dict(lse=FAKE + 2), -10),
])
def test_fwd_fp8qk_rejects(kw, code):
    assert fp8qk(**kw) == code
