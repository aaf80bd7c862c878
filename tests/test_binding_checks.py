"""The Python binding checks every tensor against the sizes it hands to the C
ABI (which sees only pointers) and raises before anything is launched.  CPU
tensors: the shape and dtype checks come before the device check, so each
case below fails on the mismatch it plants; with everything consistent the
call still stops at the device check."""
import pytest
import torch

import attention_attn_fwd_06_amd as attn

F16, BF16, F32 = torch.float16, torch.bfloat16, torch.float32


def t(*shape, dtype=F16):
    return torch.zeros(shape, dtype=dtype)


# ---- attn_fwd -------------------------------------------------------------

def fwd_args(**kw):
    a = dict(q=t(2, 64, 4, 64), k=t(2, 80, 2, 64), v=t(2, 80, 2, 64), o=None, lse=None)
    a.update(kw)
    return a


@pytest.mark.parametrize("kw,msg", [
    (dict(k=t(2, 80, 2, 64, dtype=BF16)), "k has dtype"),
    (dict(v=t(2, 80, 2, 64, dtype=BF16)), "v has dtype"),
    (dict(v=t(2, 81, 2, 64)), "v has shape"),
    (dict(k=t(3, 80, 2, 64), v=t(3, 80, 2, 64)), "k has shape"),
    (dict(k=t(2, 80, 2, 32), v=t(2, 80, 2, 32)), "k has shape"),
    (dict(o=t(2, 64, 4, 32)), "o has shape"),
    (dict(o=t(2, 64, 4, 64, dtype=BF16)), "o has dtype"),
    (dict(lse=t(2, 4, 63, dtype=F32)), "lse has shape"),
    (dict(lse=t(2, 4, 64, dtype=F16)), "lse has dtype"),
    (dict(lse=t(2, 64, 4, dtype=F32).transpose(1, 2)), "lse must be contiguous"),
    (dict(q=t(2, 64, 4, 64)[..., ::2]), "contiguous last dimension"),
])
def test_attn_fwd_rejects_mismatch(kw, msg):
    a = fwd_args(**kw)
    with pytest.raises(ValueError, match=msg):
        attn.attn_fwd(a["q"], a["k"], a["v"], o=a["o"], lse=a["lse"])


def test_attn_fwd_rejects_dtype():
    with pytest.raises(TypeError):
        attn.attn_fwd(t(1, 8, 1, 64, dtype=F32), t(1, 8, 1, 64, dtype=F32), t(1, 8, 1, 64, dtype=F32))


def test_attn_fwd_consistent_cpu_tensors_stop_at_device():
    a = fwd_args(o=t(2, 64, 4, 64), lse=t(2, 4, 64, dtype=F32))
    with pytest.raises(ValueError, match="must be a GPU tensor"):
        attn.attn_fwd(a["q"], a["k"], a["v"], o=a["o"], lse=a["lse"])


# ---- attn_decode_splitkv / fp8 ----------------------------------------------

@pytest.mark.parametrize("kw,msg", [
    (dict(k=t(1, 2, 300, 128, dtype=BF16)), "k has dtype"),
    (dict(v=t(1, 2, 299, 128)), "v has shape"),
    (dict(k=t(1, 2, 300, 64), v=t(1, 2, 300, 64)), "k has shape"),
    (dict(o_part=t(1, 8, 2, 128, dtype=F32)), "o_part has shape"),
    (dict(o_part=t(1, 8, 3, 128, dtype=F16)), "o_part has dtype"),
    (dict(lse_part=t(1, 8, 4, dtype=F32)), "lse_part has shape"),
    (dict(chunk_size=0), "chunk_size must be positive"),
])
def test_decode_splitkv_rejects_mismatch(kw, msg):
    a = dict(q=t(1, 8, 128), k=t(1, 2, 300, 128), v=t(1, 2, 300, 128), o_part=None, lse_part=None, chunk_size=128)
    a.update(kw)
    with pytest.raises(ValueError, match=msg):
        attn.attn_decode_splitkv(a["q"], a["k"], a["v"], a["chunk_size"], o_part=a["o_part"], lse_part=a["lse_part"])


def test_decode_fp8kv_rejects_mismatch():
    q = t(1, 8, 64)
    k8 = t(1, 2, 300, 64, dtype=torch.uint8)
    with pytest.raises(TypeError):
        attn.attn_decode_fp8kv_splitkv(q, t(1, 2, 300, 64), k8, 1.0, 1.0)
    with pytest.raises(ValueError, match="v has shape"):
        attn.attn_decode_fp8kv_splitkv(q, k8, t(1, 2, 301, 64, dtype=torch.uint8), 1.0, 1.0)
    with pytest.raises(ValueError, match="lse_part has shape"):
        attn.attn_decode_fp8kv_splitkv(q, k8, k8, 1.0, 1.0, lse_part=t(1, 8, 2, dtype=F32))
    with pytest.raises(ValueError, match="must be a GPU tensor"):
        attn.attn_decode_fp8kv_splitkv(q, k8, k8, 1.0, 1.0)


def test_decode_fp8kv_fused_rejects_mismatch():
    q = t(1, 8, 64)
    k8 = t(1, 2, 300, 64, dtype=torch.uint8)
    with pytest.raises(TypeError):
        attn.attn_decode_fp8kv_fused(q, t(1, 2, 300, 64), k8, 1.0, 1.0)
    with pytest.raises(ValueError, match="v has shape"):
        attn.attn_decode_fp8kv_fused(q, k8, t(1, 2, 301, 64, dtype=torch.uint8), 1.0, 1.0)
    with pytest.raises(ValueError, match="o has dtype"):
        attn.attn_decode_fp8kv_fused(q, k8, k8, 1.0, 1.0, o=t(1, 8, 64, dtype=BF16))
    with pytest.raises(ValueError, match="lse has shape"):
        attn.attn_decode_fp8kv_fused(q, k8, k8, 1.0, 1.0, lse=t(1, 4, dtype=F32))
    with pytest.raises(ValueError, match="workspace holds"):
        attn.attn_decode_fp8kv_fused(q, k8, k8, 1.0, 1.0, workspace=t(16, dtype=torch.uint8))
    with pytest.raises(ValueError, match="must be a GPU tensor"):
        attn.attn_decode_fp8kv_fused(q, k8, k8, 1.0, 1.0)


# ---- paged ------------------------------------------------------------------

def paged_args(**kw):
    a = dict(q=t(2, 8, 64), kc=t(10, 16, 2, 64), vc=t(10, 16, 2, 64),
             table=torch.zeros((2, 4), dtype=torch.int32), lens=torch.zeros(2, dtype=torch.int32),
             o_part=None, lse_part=None, k_scale=None, v_scale=None)
    a.update(kw)
    return a


def call_paged(a):
    return attn.attn_decode_paged_splitkv(a["q"], a["kc"], a["vc"], a["table"], a["lens"], 128,
                                          o_part=a["o_part"], lse_part=a["lse_part"],
                                          k_scale=a["k_scale"], v_scale=a["v_scale"])


@pytest.mark.parametrize("kw,msg", [
    (dict(kc=t(10, 16, 2, 64, dtype=BF16), vc=t(10, 16, 2, 64, dtype=BF16)), "k_cache has dtype"),
    (dict(vc=t(10, 16, 2, 32)), "same shape and strides"),
    (dict(kc=t(10, 16, 2, 32), vc=t(10, 16, 2, 32)), "shape mismatch"),
    (dict(table=torch.zeros((3, 4), dtype=torch.int32)), "shape mismatch"),
    (dict(table=torch.zeros((2, 4), dtype=torch.int64)), "block_table must be"),
    (dict(lens=torch.zeros(3, dtype=torch.int32)), "shape mismatch"),
    (dict(o_part=t(2, 8, 2, 64, dtype=F32)), "o_part has shape"),
    (dict(kc=t(10, 16, 2, 64, dtype=torch.uint8), vc=t(10, 16, 2, 64, dtype=torch.uint8)), "need k_scale"),
    (dict(kc=t(10, 16, 2, 64, dtype=torch.uint8), k_scale=1.0, v_scale=1.0), "v_cache must too"),
])
def test_paged_rejects_mismatch(kw, msg):
    with pytest.raises(ValueError, match=msg):
        call_paged(paged_args(**kw))


def test_paged_consistent_cpu_tensors_stop_at_device():
    with pytest.raises(ValueError, match="must be a GPU tensor"):
        call_paged(paged_args())


def test_paged_fused_rejects_mismatch():
    a = paged_args(kc=t(10, 16, 2, 64, dtype=torch.uint8), vc=t(10, 16, 2, 64, dtype=torch.uint8))
    with pytest.raises(ValueError, match="need k_scale"):
        attn.attn_decode_paged_fused(a["q"], a["kc"], a["vc"], a["table"], a["lens"])
    with pytest.raises(ValueError, match="o has shape"):
        attn.attn_decode_paged_fused(a["q"], a["kc"], a["vc"], a["table"], a["lens"], o=t(2, 8, 32),
                                     k_scale=1.0, v_scale=1.0)
    with pytest.raises(ValueError, match="must be a GPU tensor"):
        attn.attn_decode_paged_fused(a["q"], a["kc"], a["vc"], a["table"], a["lens"], k_scale=1.0, v_scale=1.0)


# ---- lse_merge ----------------------------------------------------------------

@pytest.mark.parametrize("kw,msg", [
    (dict(lse_part=t(2, 3, 4, dtype=F32)), "lse_part has shape"),
    (dict(lse_part=t(2, 3, 5, dtype=F16)), "lse_part has dtype"),
    (dict(o_part=t(2, 3, 5, 64)), "o_part has dtype"),
    (dict(o=t(2, 3, 32)), "o has shape"),
    (dict(lse=t(2, 4, dtype=F32)), "lse has shape"),
])
def test_lse_merge_rejects_mismatch(kw, msg):
    a = dict(o_part=t(2, 3, 5, 64, dtype=F32), lse_part=t(2, 3, 5, dtype=F32), o=None, lse=None)
    a.update(kw)
    with pytest.raises(ValueError, match=msg):
        attn.lse_merge(a["o_part"], a["lse_part"], o=a["o"], lse=a["lse"])


def test_lse_merge_consistent_cpu_tensors_stop_at_device():
    with pytest.raises(ValueError, match="must be a GPU tensor"):
        attn.lse_merge(t(2, 3, 5, 64, dtype=F32), t(2, 3, 5, dtype=F32), o=t(2, 3, 64), lse=t(2, 3, dtype=F32))
