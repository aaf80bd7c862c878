"""GPU path against the CPU oracle, through the C ABI (needs an MI355X).

Tolerances (fixed for this method): max|dO| <= 2e-3 for fp16 and <= 8e-3 for
bf16 outputs, |dlse| <= 1e-3, both against the unrounded float64 oracle on the
same seeded, already-rounded inputs.  Decode partials (fp32) are held to the
same bounds.
"""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import oracle
from tests.rescale_emu import rescale_events
from tests.test_rescale_cases import RESCALE_CASES, check_case_events, rescale_case_inputs
from workloads import WORKLOADS, decode_inputs, make_inputs, prefill_fp8qk_inputs, prefill_inputs, torch_dtype

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

DEV = "cuda"
TOL_O = {"f16": 2e-3, "bf16": 8e-3}
TOL_LSE = 1e-3


def attn():
    import attention_attn_fwd_06_amd as a
    return a


def say(msg):
    print(msg, flush=True)


def f64(t):
    return t.detach().float().cpu().double().numpy()


def maxerr(a, b):
    return float(np.max(np.abs(np.asarray(a, np.float64) - np.asarray(b, np.float64))))


def gpu_fwd(q, k, v, causal, scale):
    o, lse = attn().attn_fwd(q.to(DEV), k.to(DEV), v.to(DEV), causal=causal, scale=scale)
    torch.cuda.synchronize()
    return f64(o), f64(lse)


def check_prefill(q, k, v, causal, scale, dtype, rows=None, bh=None, label=""):
    """Run the GPU on the whole problem; compare all of it, or the given
    (batch, head) pairs and query rows, with the oracle."""
    Og, Lg = gpu_fwd(q, k, v, causal, scale)
    assert np.all(np.isfinite(Og)) and np.all(np.isfinite(Lg)), "non-finite output"
    if bh is None:
        Or, Lr = oracle.attn_ref(q, k, v, scale, causal)
        eo, el = maxerr(Og, Or), maxerr(Lg, Lr)
    else:
        Hq, Hkv = q.shape[2], k.shape[2]
        eo = el = 0.0
        for b, h in bh:
            kh = h // (Hq // Hkv)
            Or, Lr = oracle.attn_ref(q[b:b + 1, :, h:h + 1], k[b:b + 1, :, kh:kh + 1],
                                     v[b:b + 1, :, kh:kh + 1], scale, causal, rows=rows)
            eo = max(eo, maxerr(Og[b:b + 1, rows, h:h + 1], Or))
            el = max(el, maxerr(Lg[b:b + 1, h:h + 1, rows], Lr))
    say(f"  {label}: max|dO|={eo:.3e} max|dlse|={el:.3e}")
    assert eo <= TOL_O[dtype], f"{label}: max|dO| {eo:.3e} > {TOL_O[dtype]}"
    assert el <= TOL_LSE, f"{label}: max|dlse| {el:.3e} > {TOL_LSE}"


# --------------------------------------------------------------------------
# prefill
# --------------------------------------------------------------------------

def test_prefill_tiny_workload_whole():
    w = WORKLOADS["tiny_mha_fp16_d64"]
    say(f"case {w.name}")
    q, k, v = make_inputs(w, 0)
    check_prefill(q, k, v, w.causal, w.scale, w.dtype, label=w.name)


SHAPES = [
    # B, N, M, Hq, Hkv, d, dtype, causal
    (1, 1, 1, 1, 1, 64, "f16", False),
    (1, 1, 1, 2, 1, 128, "bf16", True),
    (1, 200, 333, 4, 4, 64, "f16", False),
    (1, 130, 70, 2, 2, 64, "bf16", False),
    (2, 256, 256, 4, 1, 128, "f16", True),
    (1, 520, 520, 8, 2, 128, "bf16", True),
    (3, 97, 97, 4, 4, 64, "bf16", True),
    (1, 64, 4096, 8, 8, 128, "f16", False),
    (2, 384, 384, 8, 4, 64, "f16", True),
    (1, 300, 300, 16, 2, 128, "bf16", False),
    (1, 129, 129, 8, 8, 128, "f16", True),
    # GQA groups and KV-head counts that are not powers of two (grid decode)
    (2, 300, 300, 6, 3, 128, "bf16", True),
    (1, 257, 257, 6, 2, 64, "f16", True),
    # causal with N < M: the queries are the last N positions (bottom-right mask)
    (1, 1, 333, 4, 2, 128, "bf16", True),
    (2, 64, 200, 8, 2, 128, "bf16", True),
    (1, 100, 1000, 4, 1, 64, "f16", True),
    (1, 130, 515, 8, 8, 128, "f16", True),
    # head dim 32 (the pages' smallest supported head dim)
    (1, 200, 333, 4, 4, 32, "f16", False),
    (2, 300, 300, 8, 2, 32, "bf16", True),
    (1, 70, 530, 4, 1, 32, "f16", True),
    (1, 1, 1, 1, 1, 32, "bf16", False),
    # head dim 256 (one wave per SIMD, 128 KB of K/V tiles)
    (1, 200, 333, 4, 4, 256, "f16", False),
    (2, 300, 300, 8, 2, 256, "bf16", True),
    (1, 64, 530, 4, 1, 256, "bf16", True),
    (1, 1, 1, 1, 1, 256, "f16", True),
    (1, 1024, 1024, 4, 2, 256, "bf16", True),
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_prefill_shapes_whole(shape):
    B, N, M, Hq, Hkv, d, dt, causal = shape
    say(f"case prefill {shape}")
    g = torch.Generator("cpu").manual_seed(1234 + N + M)
    q = torch.randn((B, N, Hq, d), generator=g).to(torch_dtype(dt))
    k = torch.randn((B, M, Hkv, d), generator=g).to(torch_dtype(dt))
    v = torch.randn((B, M, Hkv, d), generator=g).to(torch_dtype(dt))
    check_prefill(q, k, v, causal, float(np.float32(d ** -0.5)), dt, label=str(shape))


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_prefill_causal_gqa_bf16_reduced(seed):
    """The causal GQA bf16 d=128 workload at reduced length (all rows, all
    heads): includes the early causal rows where |O| is largest."""
    say(f"case causal gqa bf16 reduced seed {seed}")
    q, k, v = prefill_inputs(2, 8, 2, 1024, 1024, 128, "bf16", seed)
    check_prefill(q, k, v, True, WORKLOADS["prefill_causal_gqa_bf16_d128"].scale, "bf16",
                  label=f"B2 Hq8 Hkv2 N1024 seed{seed}")


def test_prefill_mha_fp16_d64_full_size_whole():
    """The non-causal MHA fp16 d=64 workload at full size, every (batch, head)
    and every row against the oracle."""
    w = WORKLOADS["prefill_mha_fp16_d64"]
    say(f"case {w.name} (full size, whole output)")
    q, k, v = make_inputs(w, 0)
    check_prefill(q, k, v, w.causal, w.scale, w.dtype, label=w.name)


def test_prefill_causal_gqa_bf16_full_size_whole():
    """The causal GQA bf16 d=128 workload at full size, every (batch, head)
    and every row against the oracle (its largest |O| outside row 0 is about
    3.2, where the bf16 output's own rounding is up to 7.8e-3)."""
    w = WORKLOADS["prefill_causal_gqa_bf16_d128"]
    say(f"case {w.name} (full size, whole output)")
    q, k, v = make_inputs(w, 0)
    check_prefill(q, k, v, w.causal, w.scale, w.dtype, label=w.name)


@pytest.mark.parametrize("case", RESCALE_CASES, ids=lambda c: "x".join(map(str, c)))
def test_prefill_rescale_branch(case):
    """Scores that grow with the key index, so that rows' maxima rise by more
    than 8 log2 units from tile to tile: the kernel moves its reference max
    (O and l rescaled by alpha = 2^(m_old - m_new)): its max-free pass keeps
    weights far above the reference, or is rerun with the exact steps, which
    rescale on the steady-state and the general path (all checked on the
    host first); and the output still matches the oracle element by
    element."""
    B, N, M, Hq, Hkv, d, dt, causal = case[:8]
    say(f"case prefill rescale {case}")
    q, k, v, scale = rescale_case_inputs(case)
    ev = rescale_events(q, k, scale, causal, max_free=True, p_dtype=dt)
    check_case_events(case, ev)
    say(f"  rescale events: steady-state {ev['fast']}, general {ev['general']}, max-free kept "
        f"{ev['free_growth']}, rerun {ev['restart']}, largest jump {ev['max_jump']:.1f}")
    check_prefill(q, k, v, causal, scale, dt, label=f"rescale {case}")


# FP8 Q and K (E4M3 codes, per-tensor scales), 16-bit V: the oracle is the
# attention of the decoded values times the scales
FP8QK_SHAPES = [
    # B, N, M, Hq, Hkv, d, dtype (of v and o), causal
    (1, 128, 128, 2, 2, 64, "f16", False),
    (2, 300, 300, 8, 2, 128, "bf16", True),
    (1, 257, 257, 6, 2, 64, "bf16", True),
    (1, 200, 333, 4, 4, 128, "f16", False),
    (2, 64, 200, 8, 2, 128, "bf16", True),
    (1, 1, 1, 1, 1, 64, "f16", False),
    (2, 1024, 1024, 8, 2, 128, "bf16", True),
]


@pytest.mark.parametrize("shape", FP8QK_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_prefill_fp8qk(shape):
    B, N, M, Hq, Hkv, d, dt, causal = shape
    say(f"case fp8 qk prefill {shape}")
    q8, k8, v, qs, ks = prefill_fp8qk_inputs(B, Hq, Hkv, N, M, d, dt, seed=N + M + d)
    scale = float(np.float32(d ** -0.5))
    o, lse = attn().attn_fwd_fp8qk(q8.to(DEV), k8.to(DEV), v.to(DEV), qs, ks, causal=causal, scale=scale)
    torch.cuda.synchronize()
    Or, Lr = oracle.attn_fp8qk_ref(q8.numpy(), k8.numpy(), v, qs, ks, scale, causal)
    eo, el = maxerr(f64(o), Or), maxerr(f64(lse), Lr)
    say(f"  max|dO|={eo:.3e} max|dlse|={el:.3e}")
    assert eo <= TOL_O[dt] and el <= TOL_LSE


def test_prefill_fp8qk_causal_gqa_full_size_whole():
    """The causal GQA d=128 workload's shape with FP8 Q and K, whole output."""
    w = WORKLOADS["prefill_causal_gqa_bf16_d128"]
    say("case fp8 qk prefill, causal GQA workload shape (whole output)")
    q8, k8, v, qs, ks = prefill_fp8qk_inputs(w.B, w.Hq, w.Hkv, w.N, w.M, w.d, "bf16", seed=0)
    o, lse = attn().attn_fwd_fp8qk(q8.to(DEV), k8.to(DEV), v.to(DEV), qs, ks, causal=True, scale=w.scale)
    torch.cuda.synchronize()
    Or, Lr = oracle.attn_fp8qk_ref(q8.numpy(), k8.numpy(), v, qs, ks, w.scale, True)
    eo, el = maxerr(f64(o), Or), maxerr(f64(lse), Lr)
    say(f"  max|dO|={eo:.3e} max|dlse|={el:.3e}")
    assert eo <= TOL_O["bf16"] and el <= TOL_LSE


def test_prefill_causal_chunk_matches_full_rows():
    """A causal chunk of the last N queries against all M keys gives the same
    rows as the full-length causal call, to the parity bound (the two calls
    tile the rows differently, so bitwise equality is not expected)."""
    say("case causal chunk vs full rows")
    q, k, v = prefill_inputs(1, 8, 2, 700, 700, 128, "bf16", 8)
    scale = float(np.float32(128 ** -0.5))
    Of, Lf = gpu_fwd(q, k, v, True, scale)
    for n in (1, 77, 300):
        Oc, Lc = gpu_fwd(q[:, 700 - n:].contiguous(), k, v, True, scale)
        assert maxerr(Oc, Of[:, 700 - n:]) <= 2 * TOL_O["bf16"], n
        assert maxerr(Lc, Lf[:, :, 700 - n:]) <= 2 * TOL_LSE, n


def test_prefill_strided_layouts():
    """Strided views through attn_fwd_strided: q, k, v as slices of one fused
    [B, N, 3, H, d] projection; head-major [B, H, N, d] tensors transposed to
    [B, N, H, d] with a head-major output; results equal the contiguous call
    bit for bit (the same kernel work per (batch, head))."""
    say("case prefill strided layouts")
    g = torch.Generator("cpu").manual_seed(4321)
    B, N, H, d = 2, 333, 4, 128
    qkv = torch.randn((B, N, 3, H, d), generator=g).to(torch.bfloat16).to(DEV)
    q, k, v = qkv[:, :, 0], qkv[:, :, 1], qkv[:, :, 2]
    assert not q.is_contiguous()
    scale = float(np.float32(d ** -0.5))
    for causal in (False, True):
        o_s, l_s = attn().attn_fwd(q, k, v, causal=causal, scale=scale)
        o_c, l_c = attn().attn_fwd(q.contiguous(), k.contiguous(), v.contiguous(), causal=causal, scale=scale)
        torch.cuda.synchronize()
        assert torch.equal(o_s, o_c) and torch.equal(l_s, l_c), causal
        Or, Lr = oracle.attn_ref(q.cpu(), k.cpu(), v.cpu(), scale, causal)
        assert maxerr(f64(o_s), Or) <= TOL_O["bf16"] and maxerr(f64(l_s), Lr) <= TOL_LSE
    # head-major storage, GQA, fp16, d = 64, N < M causal, head-major output
    Hq, Hkv, N, M, d = 8, 2, 200, 264, 64
    qh = torch.randn((1, Hq, N, d), generator=g).to(torch.float16).to(DEV)
    kh = torch.randn((1, Hkv, M, d), generator=g).to(torch.float16).to(DEV)
    vh = torch.randn((1, Hkv, M, d), generator=g).to(torch.float16).to(DEV)
    oh = torch.empty((1, Hq, N, d), dtype=torch.float16, device=DEV)
    q, k, v, o = (t.transpose(1, 2) for t in (qh, kh, vh, oh))
    attn().attn_fwd(q, k, v, causal=True, scale=0.125, o=o)
    o_c, _ = attn().attn_fwd(q.contiguous(), k.contiguous(), v.contiguous(), causal=True, scale=0.125)
    torch.cuda.synchronize()
    assert torch.equal(oh.transpose(1, 2), o_c)
    Or, _ = oracle.attn_ref(q.cpu(), k.cpu(), v.cpu(), 0.125, True)
    assert maxerr(f64(o), Or) <= TOL_O["f16"]


def test_prefill_q_beyond_2_31_elements():
    """q and o of 2^31 elements (4 GiB each): rows past the 2^31st element
    are read and written through 64-bit offsets.  Checked against the oracle
    on the last rows of every head."""
    B, N, Hq, Hkv, M, d = 1, 262144, 64, 1, 128, 128
    say(f"case prefill q with {B * N * Hq * d} elements")
    g = torch.Generator("cpu").manual_seed(31)
    k = torch.randn((B, M, Hkv, d), generator=g).to(torch.bfloat16)
    v = torch.randn((B, M, Hkv, d), generator=g).to(torch.bfloat16)
    q = torch.empty((B, N, Hq, d), dtype=torch.bfloat16, device=DEV)
    q.normal_(generator=torch.Generator(DEV).manual_seed(32))
    scale = float(np.float32(d ** -0.5))
    o, lse = attn().attn_fwd(q, k.to(DEV), v.to(DEV), causal=False, scale=scale)
    torch.cuda.synchronize()
    rows = np.arange(N - 40, N)
    qs = q[:, N - 40:].cpu()
    Or, Lr = oracle.attn_ref(qs, k, v, scale, False)
    eo = maxerr(f64(o[:, N - 40:]), Or)
    el = maxerr(f64(lse[:, :, N - 40:]), Lr)
    say(f"  last rows: max|dO|={eo:.3e} max|dlse|={el:.3e}")
    assert eo <= TOL_O["bf16"] and el <= TOL_LSE
    del q, o, lse
    torch.cuda.empty_cache()


def test_prefill_deterministic():
    say("case prefill determinism")
    q, k, v = prefill_inputs(1, 8, 2, 520, 520, 128, "bf16", 5)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    o1, l1 = attn().attn_fwd(qd, kd, vd, causal=True)
    o2, l2 = attn().attn_fwd(qd, kd, vd, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_prefill_writes_every_output():
    say("case prefill NaN-poisoned outputs")
    q, k, v = prefill_inputs(2, 4, 2, 333, 333, 64, "f16", 6)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    o = torch.full_like(qd, float("nan"))
    lse = torch.full((2, 4, 333), float("nan"), device=DEV)
    attn().attn_fwd(qd, kd, vd, causal=True, o=o, lse=lse)
    torch.cuda.synchronize()
    assert not torch.isnan(o).any() and not torch.isnan(lse).any()


def test_prefill_invariants_black_box():
    say("case prefill invariants")
    B, N, Hq, Hkv, d = 1, 200, 8, 2, 128
    q, k, v = prefill_inputs(B, Hq, Hkv, N, N, d, "bf16", 7)
    scale = float(np.float32(d ** -0.5))
    # constant V rows -> O equals that row
    u = v[:, :1].expand_as(v).contiguous()
    Og, _ = gpu_fwd(q, k, u, True, scale)
    ref = np.broadcast_to(f64(u[:, :1]).repeat(Hq // Hkv, axis=2), Og.shape)
    assert maxerr(Og, ref) <= TOL_O["bf16"]
    # causal row 0 is exactly V[0] of its KV head
    Og, Lg = gpu_fwd(q, k, v, True, scale)
    v0 = f64(v[:, 0]).repeat(Hq // Hkv, axis=1)
    assert maxerr(Og[:, 0], v0) == 0.0
    # GQA == MHA with repeated KV heads (same kernel work per head: bitwise)
    kr = k.repeat_interleave(Hq // Hkv, dim=2).contiguous()
    vr = v.repeat_interleave(Hq // Hkv, dim=2).contiguous()
    Og2, Lg2 = gpu_fwd(q, kr, vr, True, scale)
    assert np.array_equal(Og, Og2) and np.array_equal(Lg, Lg2)
    # scale = 0: uniform weights, lse = ln(#allowed keys)
    Og, Lg = gpu_fwd(q, k, v, True, 0.0)
    cnt = np.arange(1, N + 1)
    assert maxerr(Lg, np.broadcast_to(np.log(cnt), Lg.shape)) <= TOL_LSE
    vf = f64(v).repeat(Hq // Hkv, axis=2)
    ref = np.cumsum(vf, axis=1) / cnt[None, :, None, None]
    assert maxerr(Og, ref) <= TOL_O["bf16"]


# --------------------------------------------------------------------------
# decode
# --------------------------------------------------------------------------

def gpu_decode(q, k, v, chunk, scale):
    o, lse, op, lp = attn().attn_decode(q.to(DEV), k.to(DEV), v.to(DEV), chunk, scale)
    torch.cuda.synchronize()
    return f64(o), f64(lse), f64(op), f64(lp)


def check_decode(q, k, v, chunk, scale, dtype, label):
    Og, Lg, OPg, LPg = gpu_decode(q, k, v, chunk, scale)
    Or, Lr, OPr, LPr = oracle.decode_ref(q, k, v, scale, chunk)
    errs = dict(o=maxerr(Og, Or), lse=maxerr(Lg, Lr), o_part=maxerr(OPg, OPr), lse_part=maxerr(LPg, LPr))
    say(f"  {label}: " + " ".join(f"{n}={e:.3e}" for n, e in errs.items()))
    assert errs["o"] <= TOL_O[dtype] and errs["o_part"] <= TOL_O[dtype], errs
    assert errs["lse"] <= TOL_LSE and errs["lse_part"] <= TOL_LSE, errs


@pytest.mark.parametrize("name", ["small_decode_fp16_d128", "long_decode_fp16_d128", "gqa_decode_bf16_d128"])
def test_decode_workload_whole(name):
    w = WORKLOADS[name]
    say(f"case {w.name}")
    q, k, v = make_inputs(w, 0)
    check_decode(q, k, v, w.chunk, w.scale, w.dtype, w.name)


DEC_SHAPES = [
    # B, Hq, Hkv, M, d, dtype
    (1, 1, 1, 1, 128, "f16"),
    (1, 2, 1, 127, 64, "f16"),
    (2, 8, 2, 1000, 128, "bf16"),
    (1, 4, 4, 129, 64, "bf16"),
    (3, 16, 4, 4096, 128, "f16"),
    # GQA groups of 3, 6, 8 and 16: one item serves 1, 2, 4 and 4 query heads
    (2, 24, 8, 777, 128, "bf16"),
    (1, 12, 2, 300, 64, "f16"),
    (2, 32, 4, 2049, 128, "bf16"),
    (1, 16, 1, 513, 64, "bf16"),
    # larger MHA launches, one with a tail chunk
    (2, 8, 8, 16461, 64, "f16"),
    (1, 16, 16, 16384, 128, "bf16"),
    # groups split over several 16-column slices: 32 = 2 x 16, 24 = 2 x 12
    (1, 32, 1, 300, 128, "bf16"),
    (2, 24, 1, 200, 64, "f16"),
    # head dim 32: VALU (small MHA), matrix-core (GQA and large MHA)
    (1, 4, 4, 300, 32, "f16"),
    (2, 16, 4, 1000, 32, "bf16"),
    (4, 8, 8, 8200, 32, "f16"),
    # head dim 256 (matrix-core kernel for every launch; 8-row fetch instructions)
    (1, 4, 4, 300, 256, "f16"),
    (2, 16, 4, 1000, 256, "bf16"),
    (1, 8, 8, 2100, 256, "bf16"),
    (1, 24, 8, 777, 256, "f16"),
]


@pytest.mark.parametrize("shape", DEC_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_decode_shapes(shape):
    B, Hq, Hkv, M, d, dt = shape
    say(f"case decode {shape}")
    q, k, v = decode_inputs(B, Hq, Hkv, M, d, dt, seed=M)
    check_decode(q, k, v, 128, float(np.float32(d ** -0.5)), dt, str(shape))


def test_decode_kv_slice_beyond_2_31_bytes():
    """One (batch, kv head) slice of K and V of 8.4M keys (2.1 GB each, past
    2^31 bytes; the kernels address a slice with 32-bit buffer offsets),
    through the two-launch and the one-launch decode.  The oracle runs over
    ranges of whole chunks (a chunk's partial depends only on its own keys)
    and merges all partials once, so the whole output is compared."""
    B, Hq, Hkv, d, dt, chunk = 1, 2, 1, 128, "bf16", 1024
    M = (1 << 23) + 77
    say(f"case decode with a {M}-key slice")
    q, k, v = decode_inputs(B, Hq, Hkv, M, d, dt, seed=5, device=DEV)
    scale = float(np.float32(d ** -0.5))
    o, lse, op, lp = attn().attn_decode(q, k, v, chunk, scale)
    of, lf = attn().attn_decode_fused(q, k, v, scale)
    torch.cuda.synchronize()
    C = -(-M // chunk)
    qc, parts_o, parts_l = q.cpu(), [], []
    step = 1024                                   # chunks per oracle call
    for c0 in range(0, C, step):
        lo, hi = c0 * chunk, min(M, (c0 + step) * chunk)
        po, pl = oracle.decode_partials_ref(qc, k[:, :, lo:hi].cpu(), v[:, :, lo:hi].cpu(), scale, chunk)
        parts_o.append(po)
        parts_l.append(pl)
    OPr, LPr = np.concatenate(parts_o, axis=2), np.concatenate(parts_l, axis=2)
    Or, Lr = oracle.lse_merge_ref(OPr, LPr)
    errs = dict(o=maxerr(f64(o), Or), lse=maxerr(f64(lse), Lr), o_part=maxerr(f64(op), OPr),
                lse_part=maxerr(f64(lp), LPr), o_fused=maxerr(f64(of), Or), lse_fused=maxerr(f64(lf), Lr))
    say("  " + " ".join(f"{n}={e:.3e}" for n, e in errs.items()))
    assert max(errs["o"], errs["o_part"], errs["o_fused"]) <= TOL_O[dt], errs
    assert max(errs["lse"], errs["lse_part"], errs["lse_fused"]) <= TOL_LSE, errs


# chunks longer than 128 keys (walked as 128-key sub-chunks with the online
# rescale between them), with short last chunks and sub-chunks
@pytest.mark.parametrize("shape", [(1, 8, 2, 1000, 128, "bf16", 256), (2, 4, 4, 3000, 64, "f16", 512),
                                   (1, 16, 2, 777, 128, "f16", 1024), (1, 4, 1, 9000, 64, "bf16", 8192),
                                   (2, 8, 8, 2049, 128, "f16", 384), (1, 32, 4, 130, 128, "bf16", 8192),
                                   (1, 8, 2, 2000, 32, "bf16", 512), (1, 8, 2, 1000, 256, "bf16", 512)],
                         ids=lambda s: "x".join(map(str, s)))
def test_decode_chunk_sizes(shape):
    B, Hq, Hkv, M, d, dt, chunk = shape
    say(f"case decode chunk {shape}")
    q, k, v = decode_inputs(B, Hq, Hkv, M, d, dt, seed=M + chunk)
    check_decode(q, k, v, chunk, float(np.float32(d ** -0.5)), dt, str(shape))


# paged KV cache: shuffled pages, NaN in every row no sequence owns (rows past
# a sequence's end inside its last page, and spare pages), table slots past a
# sequence holding -1 or out-of-range ids, so a stray read shows up as NaN
def paged_inputs(B, Hq, Hkv, lens, d, dt, bs, seed, head_major):
    M = max(lens)
    q, k, v = decode_inputs(B, Hq, Hkv, M, d, dt, seed=seed)
    nblk = [-(-n // bs) for n in lens]
    max_blocks = max(nblk) + 1
    total = sum(nblk) + 3
    order = torch.randperm(total, generator=torch.Generator().manual_seed(seed)).tolist()
    tdt = torch_dtype(dt)
    shape = (total, Hkv, bs, d) if head_major else (total, bs, Hkv, d)
    kc = torch.full(shape, float("nan"), dtype=tdt)
    vc = torch.full(shape, float("nan"), dtype=tdt)
    kv_k = kc.transpose(1, 2) if head_major else kc   # [pages, bs, Hkv, d] views
    kv_v = vc.transpose(1, 2) if head_major else vc
    table = torch.full((B, max_blocks), -1, dtype=torch.int32)
    nxt = 0
    for b in range(B):
        for j in range(nblk[b]):
            pg = order[nxt]
            nxt += 1
            table[b, j] = pg
            lo, hi = j * bs, min((j + 1) * bs, lens[b])
            kv_k[pg, :hi - lo] = k[b, :, lo:hi].transpose(0, 1)
            kv_v[pg, :hi - lo] = v[b, :, lo:hi].transpose(0, 1)
        if nblk[b] < max_blocks:
            table[b, nblk[b]] = total + 5 if b % 2 else -1
    return q, kc, vc, kv_k, kv_v, table, torch.tensor(lens, dtype=torch.int32)


PAGED_CASES = [
    # B, Hq, Hkv, lens, d, dtype, block_size, chunk, head_major
    (3, 8, 2, (1, 200, 1000), 128, "bf16", 16, 128, False),
    (2, 4, 4, (777, 64), 64, "f16", 64, 256, True),
    (4, 32, 8, (5000, 3, 128, 4097), 128, "f16", 256, 512, False),
    (2, 16, 1, (130, 16), 32, "bf16", 32, 128, True),
    (1, 2, 1, (2048,), 128, "f16", 128, 128, False),
    (2, 12, 4, (300, 2000), 64, "bf16", 48, 1024, False),
    (2, 8, 2, (300, 1000), 256, "bf16", 16, 128, False),
    (1, 4, 1, (777,), 256, "f16", 64, 256, True),
]


@pytest.mark.parametrize("case", PAGED_CASES, ids=lambda c: "x".join(map(str, c)).replace(" ", ""))
def test_decode_paged(case):
    B, Hq, Hkv, lens, d, dt, bs, chunk, head_major = case
    say(f"case paged decode {case}")
    q, kc, vc, kv_k, kv_v, table, sl = paged_inputs(B, Hq, Hkv, list(lens), d, dt, bs, seed=sum(lens), head_major=head_major)
    scale = float(np.float32(d ** -0.5))
    kd, vd = kc.to(DEV), vc.to(DEV)
    kvk_d = kd.transpose(1, 2) if head_major else kd
    kvv_d = vd.transpose(1, 2) if head_major else vd
    o, lse, op, lp = attn().attn_decode_paged(q.to(DEV), kvk_d, kvv_d, table.to(DEV), sl.to(DEV), chunk, scale)
    torch.cuda.synchronize()
    Or, Lr, OPr, LPr = oracle.paged_decode_ref(q, kv_k, kv_v, table.clamp(min=0), sl, scale, chunk)
    OPg, LPg = f64(op), f64(lp)
    full = np.isfinite(LPr)
    assert np.array_equal(np.isfinite(LPg), full), "empty chunks must be exactly the chunks past each end"
    assert np.all(OPg[~full] == 0.0)
    errs = dict(o=maxerr(f64(o), Or), lse=maxerr(f64(lse), Lr),
                o_part=maxerr(OPg[full], OPr[full]), lse_part=maxerr(LPg[full], LPr[full]))
    say(f"  {case}: " + " ".join(f"{n}={e:.3e}" for n, e in errs.items()))
    assert errs["o"] <= TOL_O[dt] and errs["o_part"] <= TOL_O[dt], errs
    assert errs["lse"] <= TOL_LSE and errs["lse_part"] <= TOL_LSE, errs


# the paged decode in one launch: the same cases (any chunk size runs as 128-key
# chunks), an empty sequence, a bad page id inside a sequence, head dim 256
PAGED_FUSED_CASES = [c for c in PAGED_CASES] + [
    (4, 16, 4, (0, 1, 4096, 700), 128, "bf16", 16, 128, False),
    (8, 8, 8, (3000,) * 8, 64, "f16", 32, 128, True),
]


@pytest.mark.parametrize("case", PAGED_FUSED_CASES, ids=lambda c: "x".join(map(str, c)).replace(" ", ""))
def test_decode_paged_fused(case):
    B, Hq, Hkv, lens, d, dt, bs, _, head_major = case
    say(f"case paged fused decode {case}")
    q, kc, vc, kv_k, kv_v, table, sl = paged_inputs(B, Hq, Hkv, list(lens), d, dt, bs, seed=sum(lens) + 1,
                                                    head_major=head_major)
    scale = float(np.float32(d ** -0.5))
    kd, vd = kc.to(DEV), vc.to(DEV)
    kvk_d = kd.transpose(1, 2) if head_major else kd
    kvv_d = vd.transpose(1, 2) if head_major else vd
    ws = torch.zeros(attn().attn_decode_fused_workspace_bytes(B, Hq, Hkv, table.shape[1] * bs, d), dtype=torch.uint8,
                     device=DEV)
    for rep in range(2):       # the second call reuses the workspace (its counters reset themselves)
        o, lse = attn().attn_decode_paged_fused(q.to(DEV), kvk_d, kvv_d, table.to(DEV), sl.to(DEV), scale,
                                                workspace=ws)
        torch.cuda.synchronize()
        Or, Lr, _, _ = oracle.paged_decode_ref(q, kv_k, kv_v, table.clamp(min=0), sl, scale, 128)
        Og, Lg = f64(o), f64(lse)
        empty = np.asarray(lens) == 0
        assert np.all(Og[empty] == 0.0) and np.all(Lg[empty] == -np.inf), "empty sequence"
        eo, el = maxerr(Og[~empty], Or[~empty]), maxerr(Lg[~empty], Lr[~empty])
        say(f"  call {rep}: o={eo:.3e} lse={el:.3e}")
        assert eo <= TOL_O[dt] and el <= TOL_LSE
    assert torch.count_nonzero(ws[:256]).item() == 0, "row counters left non-zero"


def test_decode_paged_fused_bad_page_id():
    """A page id out of range inside a sequence reads as keys and values of
    zeros, as in the two-launch paged decode."""
    B, Hq, Hkv, d, bs = 3, 8, 2, 128, 16
    lens = [5, 200, 1000]
    say("case paged fused decode, bad page id")
    q, kc, vc, kv_k, kv_v, table, sl = paged_inputs(B, Hq, Hkv, lens, d, "f16", bs, seed=78, head_major=False)
    num_blocks = kc.shape[0]
    table[2, 5] = num_blocks + 11
    scale = float(np.float32(d ** -0.5))
    o, lse = attn().attn_decode_paged_fused(q.to(DEV), kc.to(DEV), vc.to(DEV), table.to(DEV), sl.to(DEV), scale)
    torch.cuda.synchronize()
    kref, vref = f64(kc), f64(vc)
    zero = np.zeros((1,) + kref.shape[1:])
    kref, vref = np.concatenate([kref, zero]), np.concatenate([vref, zero])
    tref = table.clone()
    tref[2, 5] = num_blocks
    Or, Lr, _, _ = oracle.paged_decode_ref(q, kref, vref, tref.clamp(min=0), sl, scale, 128)
    eo, el = maxerr(f64(o), Or), maxerr(f64(lse), Lr)
    say(f"  o={eo:.3e} lse={el:.3e}")
    assert eo <= TOL_O["f16"] and el <= TOL_LSE


PAGED_FP8_CASES = [
    (3, 8, 2, (1, 200, 1000), 128, "bf16", 16, 128, False),
    (2, 4, 4, (777, 64), 64, "f16", 64, 256, True),
    (2, 16, 1, (130, 16), 32, "bf16", 32, 128, True),
    (2, 32, 8, (5000, 4097), 128, "f16", 256, 512, False),
]


@pytest.mark.parametrize("case", PAGED_FP8_CASES, ids=lambda c: "x".join(map(str, c)).replace(" ", ""))
def test_decode_paged_fp8kv(case):
    """Paged cache of E4M3 codes; the unowned rows hold NaN codes."""
    B, Hq, Hkv, lens, d, dt, bs, chunk, head_major = case
    say(f"case paged fp8 kv decode {case}")
    q, kc, vc, _, _, table, sl = paged_inputs(B, Hq, Hkv, list(lens), d, dt, bs, seed=sum(lens) + 1,
                                              head_major=head_major)
    ks, vs = float(np.float32(4.0 / 448.0)), float(np.float32(3.0 / 448.0))
    # clamp to the E4M3 range (beyond it the conversion gives NaN codes); the
    # unowned rows keep their NaN, which clamp passes through
    kc8 = (kc.float() / ks).clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8)
    vc8 = (vc.float() / vs).clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8)
    view = (lambda t: t.transpose(1, 2)) if head_major else (lambda t: t)
    scale = float(np.float32(d ** -0.5))
    kd, vd = kc8.to(DEV), vc8.to(DEV)
    o, lse, op, lp = attn().attn_decode_paged(q.to(DEV), view(kd), view(vd), table.to(DEV), sl.to(DEV), chunk, scale,
                                              k_scale=ks, v_scale=vs)
    torch.cuda.synchronize()
    kdeq = oracle.e4m3_decode(view(kc8).numpy()) * ks
    vdeq = oracle.e4m3_decode(view(vc8).numpy()) * vs
    Or, Lr, OPr, LPr = oracle.paged_decode_ref(q, kdeq, vdeq, table.clamp(min=0), sl, scale, chunk)
    OPg, LPg = f64(op), f64(lp)
    full = np.isfinite(LPr)
    assert np.array_equal(np.isfinite(LPg), full), "empty chunks must be exactly the chunks past each end"
    assert np.all(OPg[~full] == 0.0)
    errs = dict(o=maxerr(f64(o), Or), lse=maxerr(f64(lse), Lr),
                o_part=maxerr(OPg[full], OPr[full]), lse_part=maxerr(LPg[full], LPr[full]))
    say(f"  {case}: " + " ".join(f"{n}={e:.3e}" for n, e in errs.items()))
    assert errs["o"] <= TOL_O[dt] and errs["o_part"] <= TOL_O[dt], errs
    assert errs["lse"] <= TOL_LSE and errs["lse_part"] <= TOL_LSE, errs


@pytest.mark.parametrize("fp8", [False, True], ids=["f16", "fp8kv"])
def test_decode_paged_invalid_page_and_empty_sequence(fp8):
    """Sequence 0 is empty (o = 0, lse = -inf after the merge); sequence 2
    has an out-of-range page id inside its length, whose rows the kernels
    take as zero keys and values: the oracle sees the same cache with that
    id pointing at a page of zeros."""
    B, Hq, Hkv, d, bs, chunk = 3, 8, 2, 128, 16, 128
    lens = [0, 200, 1000]
    say(f"case paged decode, empty sequence and bad page id, fp8={fp8}")
    q, kc, vc, kv_k, kv_v, table, sl = paged_inputs(B, Hq, Hkv, lens, d, "f16", bs, seed=77, head_major=False)
    num_blocks = kc.shape[0]
    table[2, 5] = num_blocks + 11          # inside sequence 2 (keys 80 .. 95)
    ks, vs = float(np.float32(4.0 / 448.0)), float(np.float32(3.0 / 448.0))
    if fp8:
        kc = (kc.float() / ks).clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8)
        vc = (vc.float() / vs).clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8)
    scale = float(np.float32(d ** -0.5))
    o, lse, op, lp = attn().attn_decode_paged(q.to(DEV), kc.to(DEV), vc.to(DEV), table.to(DEV), sl.to(DEV), chunk,
                                              scale, k_scale=ks if fp8 else None, v_scale=vs if fp8 else None)
    torch.cuda.synchronize()
    if fp8:
        kref, vref = oracle.e4m3_decode(kc.numpy()) * ks, oracle.e4m3_decode(vc.numpy()) * vs
    else:
        kref, vref = f64(kc), f64(vc)
    zero = np.zeros((1,) + kref.shape[1:])
    kref, vref = np.concatenate([kref, zero]), np.concatenate([vref, zero])
    tref = table.clone()
    tref[2, 5] = num_blocks                # the appended page of zeros
    Or, Lr, OPr, LPr = oracle.paged_decode_ref(q, kref, vref, tref.clamp(min=0), sl, scale, chunk)
    Og, Lg = f64(o), f64(lse)
    assert np.all(Og[0] == 0.0) and np.all(Lg[0] == -np.inf), "empty sequence"
    assert np.all(Lr[0] == -np.inf)
    eo, el = maxerr(Og[1:], Or[1:]), maxerr(Lg[1:], Lr[1:])
    say(f"  o={eo:.3e} lse={el:.3e}")
    assert eo <= TOL_O["f16"] and el <= TOL_LSE


@pytest.mark.parametrize("dt", ["f16", "bf16"])
def test_lse_merge_empty_rows(dt):
    """Rows whose chunks are all -inf (no key) give o = 0 and lse = -inf."""
    say(f"case lse_merge empty rows {dt}")
    g = torch.Generator("cpu").manual_seed(5)
    op = torch.randn((2, 3, 40, 128), generator=g) * 0.5
    lp = torch.randn((2, 3, 40), generator=g) * 4.0
    lp[0, 1] = float("-inf")
    lp[1, 2, 7:] = float("-inf")
    op[0, 1] = 0.0
    o, lse = attn().lse_merge(op.to(DEV), lp.to(DEV), torch_dtype(dt))
    torch.cuda.synchronize()
    Or, Lr = oracle.lse_merge_ref(op, lp)
    Og, Lg = f64(o), f64(lse)
    assert np.all(Og[0, 1] == 0.0) and Lg[0, 1] == -np.inf
    fin = np.isfinite(Lr)
    assert np.array_equal(np.isfinite(Lg), fin)
    assert maxerr(Og, Or) <= TOL_O[dt] and maxerr(Lg[fin], Lr[fin]) <= TOL_LSE


def test_decode_paged_matches_contiguous():
    """One sequence in pages in order decodes like the contiguous decode."""
    say("case paged vs contiguous decode")
    B, Hq, Hkv, M, d = 2, 8, 2, 1500, 128
    q, k, v = decode_inputs(B, Hq, Hkv, M, d, "bf16", seed=21)
    bs = 32
    nb = -(-M // bs)
    pad = nb * bs - M
    kp = torch.nn.functional.pad(k, (0, 0, 0, pad)).reshape(B, Hkv, nb, bs, d).permute(0, 2, 3, 1, 4)
    vp = torch.nn.functional.pad(v, (0, 0, 0, pad)).reshape(B, Hkv, nb, bs, d).permute(0, 2, 3, 1, 4)
    kc = kp.reshape(B * nb, bs, Hkv, d).contiguous().to(DEV)
    vc = vp.reshape(B * nb, bs, Hkv, d).contiguous().to(DEV)
    table = torch.arange(B * nb, dtype=torch.int32).reshape(B, nb).to(DEV)
    sl = torch.full((B,), M, dtype=torch.int32, device=DEV)
    o1, l1, _, _ = attn().attn_decode_paged(q.to(DEV), kc, vc, table, sl, 128, 0.09)
    o2, l2, _, _ = attn().attn_decode(q.to(DEV), k.to(DEV), v.to(DEV), 128, 0.09)
    torch.cuda.synchronize()
    assert maxerr(f64(o1), f64(o2)) <= TOL_O["bf16"]
    assert maxerr(f64(l1), f64(l2)) <= TOL_LSE


# FP8 KV: K, V quantised to E4M3 codes with per-tensor scales (codes drawn by
# rounding N(0,1) values / scale to E4M3, as a caller's quantiser would)
def fp8kv_inputs(B, Hq, Hkv, M, d, dt, seed):
    q, k, v = decode_inputs(B, Hq, Hkv, M, d, dt, seed=seed)
    ks, vs = float(np.float32(4.0 / 448.0)), float(np.float32(3.0 / 448.0))
    kc = (k.float() / ks).clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8)
    vc = (v.float() / vs).clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8)
    return q, kc, vc, ks, vs


FP8_CASES = [
    # B, Hq, Hkv, M, d, dtype, chunk
    (2, 8, 2, 1000, 128, "bf16", 128),
    (1, 4, 4, 777, 64, "f16", 256),
    (2, 32, 8, 4096, 128, "f16", 512),
    (1, 16, 1, 300, 32, "bf16", 128),
    (3, 8, 8, 129, 128, "bf16", 1024),
]


@pytest.mark.parametrize("case", FP8_CASES, ids=lambda c: "x".join(map(str, c)))
def test_decode_fp8kv(case):
    B, Hq, Hkv, M, d, dt, chunk = case
    say(f"case fp8 kv decode {case}")
    q, kc, vc, ks, vs = fp8kv_inputs(B, Hq, Hkv, M, d, dt, seed=M + d)
    scale = float(np.float32(d ** -0.5))
    o, lse, op, lp = attn().attn_decode_fp8kv(q.to(DEV), kc.to(DEV), vc.to(DEV), ks, vs, chunk, scale)
    torch.cuda.synchronize()
    Or, Lr, OPr, LPr = oracle.decode_fp8kv_ref(q, kc.numpy(), vc.numpy(), ks, vs, scale, chunk)
    errs = dict(o=maxerr(f64(o), Or), lse=maxerr(f64(lse), Lr), o_part=maxerr(f64(op), OPr),
                lse_part=maxerr(f64(lp), LPr))
    say(f"  {case}: " + " ".join(f"{n}={e:.3e}" for n, e in errs.items()))
    assert errs["o"] <= TOL_O[dt] and errs["o_part"] <= TOL_O[dt], errs
    assert errs["lse"] <= TOL_LSE and errs["lse_part"] <= TOL_LSE, errs


# the FP8-KV decode in one launch (partials of 128-key chunk runs and their
# merge fused): the oracle is the two-step decode of the decoded values at
# chunk 128
FP8_FUSED_CASES = [
    # B, Hq, Hkv, M, d, dtype
    (2, 8, 2, 1000, 128, "bf16"),
    (1, 4, 4, 777, 64, "f16"),
    (8, 32, 8, 16384, 128, "bf16"),    # grouped-query decode workload
    (2, 8, 8, 65536, 128, "f16"),      # long decode shape
    (1, 16, 1, 300, 32, "bf16"),
    (3, 24, 8, 4097, 128, "f16"),      # groups of 3 heads, a one-key tail chunk
    (64, 32, 32, 1000, 64, "f16"),     # more rows than the grid: one segment per row
    (1, 1, 1, 1, 128, "bf16"),         # a single key
]


@pytest.mark.parametrize("case", FP8_FUSED_CASES, ids=lambda c: "x".join(map(str, c)))
def test_decode_fp8kv_fused(case):
    B, Hq, Hkv, M, d, dt = case
    say(f"case fp8 kv fused decode {case}")
    q, kc, vc, ks, vs = fp8kv_inputs(B, Hq, Hkv, M, d, dt, seed=M + d + 1)
    scale = float(np.float32(d ** -0.5))
    ws = torch.zeros(attn().attn_decode_fused_workspace_bytes(B, Hq, Hkv, M, d), dtype=torch.uint8, device=DEV)
    Or, Lr, _, _ = oracle.decode_fp8kv_ref(q, kc.numpy(), vc.numpy(), ks, vs, scale, 128)
    outs = []
    for rep in range(2):       # the second call reuses the workspace (its counters reset themselves)
        o, lse = attn().attn_decode_fp8kv_fused(q.to(DEV), kc.to(DEV), vc.to(DEV), ks, vs, scale, workspace=ws)
        torch.cuda.synchronize()
        eo, el = maxerr(f64(o), Or), maxerr(f64(lse), Lr)
        say(f"  call {rep}: o={eo:.3e} lse={el:.3e}")
        assert eo <= TOL_O[dt] and el <= TOL_LSE
        outs.append((o, lse))
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])
    assert torch.count_nonzero(ws[:256]).item() == 0, "row counters left non-zero"


PAGED_FP8_FUSED_CASES = [
    # B, Hq, Hkv, lens, d, dtype, block size, head-major pages
    (3, 8, 2, (1, 200, 1000), 128, "bf16", 16, False),
    (2, 4, 4, (777, 64), 64, "f16", 64, True),
    (2, 16, 1, (130, 16), 32, "bf16", 32, True),
    (2, 32, 8, (5000, 4097), 128, "f16", 256, False),
    (4, 16, 4, (0, 1, 4096, 700), 128, "bf16", 16, False),
]


@pytest.mark.parametrize("case", PAGED_FP8_FUSED_CASES, ids=lambda c: "x".join(map(str, c)).replace(" ", ""))
def test_decode_paged_fp8kv_fused(case):
    """Paged cache of E4M3 codes in one launch; the unowned rows hold NaN
    codes, an empty sequence gives o = 0 and lse = -inf."""
    B, Hq, Hkv, lens, d, dt, bs, head_major = case
    say(f"case paged fp8 kv fused decode {case}")
    q, kc, vc, _, _, table, sl = paged_inputs(B, Hq, Hkv, list(lens), d, dt, bs, seed=sum(lens) + 2,
                                              head_major=head_major)
    ks, vs = float(np.float32(4.0 / 448.0)), float(np.float32(3.0 / 448.0))
    kc8 = (kc.float() / ks).clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8)
    vc8 = (vc.float() / vs).clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8)
    view = (lambda t: t.transpose(1, 2)) if head_major else (lambda t: t)
    scale = float(np.float32(d ** -0.5))
    ws = torch.zeros(attn().attn_decode_fused_workspace_bytes(B, Hq, Hkv, table.shape[1] * bs, d), dtype=torch.uint8,
                     device=DEV)
    kdeq = oracle.e4m3_decode(view(kc8).numpy()) * ks
    vdeq = oracle.e4m3_decode(view(vc8).numpy()) * vs
    Or, Lr, _, _ = oracle.paged_decode_ref(q, kdeq, vdeq, table.clamp(min=0), sl, scale, 128)
    empty = np.asarray(lens) == 0
    for rep in range(2):
        o, lse = attn().attn_decode_paged_fused(q.to(DEV), view(kc8.to(DEV)), view(vc8.to(DEV)), table.to(DEV),
                                                sl.to(DEV), scale, workspace=ws, k_scale=ks, v_scale=vs)
        torch.cuda.synchronize()
        Og, Lg = f64(o), f64(lse)
        assert np.all(Og[empty] == 0.0) and np.all(Lg[empty] == -np.inf), "empty sequence"
        eo, el = maxerr(Og[~empty], Or[~empty]), maxerr(Lg[~empty], Lr[~empty])
        say(f"  call {rep}: o={eo:.3e} lse={el:.3e}")
        assert eo <= TOL_O[dt] and el <= TOL_LSE
    assert torch.count_nonzero(ws[:256]).item() == 0, "row counters left non-zero"


def test_decode_paged_fp8kv_fused_bad_page_id():
    """A page id out of range inside a sequence reads as keys and values of
    zeros, as in the two-launch paged FP8 decode."""
    B, Hq, Hkv, d, bs = 3, 8, 2, 128, 16
    lens = [5, 200, 1000]
    say("case paged fp8 kv fused decode, bad page id")
    q, kc, vc, _, _, table, sl = paged_inputs(B, Hq, Hkv, lens, d, "bf16", bs, seed=79, head_major=False)
    ks, vs = float(np.float32(4.0 / 448.0)), float(np.float32(3.0 / 448.0))
    kc8 = (kc.float() / ks).clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8)
    vc8 = (vc.float() / vs).clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8)
    num_blocks = kc.shape[0]
    table[2, 5] = num_blocks + 11
    scale = float(np.float32(d ** -0.5))
    o, lse = attn().attn_decode_paged_fused(q.to(DEV), kc8.to(DEV), vc8.to(DEV), table.to(DEV), sl.to(DEV), scale,
                                            k_scale=ks, v_scale=vs)
    torch.cuda.synchronize()
    kref, vref = oracle.e4m3_decode(kc8.numpy()) * ks, oracle.e4m3_decode(vc8.numpy()) * vs
    zero = np.zeros((1,) + kref.shape[1:])
    kref, vref = np.concatenate([kref, zero]), np.concatenate([vref, zero])
    tref = table.clone()
    tref[2, 5] = num_blocks
    Or, Lr, _, _ = oracle.paged_decode_ref(q, kref, vref, tref.clamp(min=0), sl, scale, 128)
    eo, el = maxerr(f64(o), Or), maxerr(f64(lse), Lr)
    say(f"  o={eo:.3e} lse={el:.3e}")
    assert eo <= TOL_O["bf16"] and el <= TOL_LSE


@pytest.mark.parametrize("dt", ["f16", "bf16"])
def test_decode_fp8kv_every_code(dt):
    """Every E4M3 code through the kernel's conversion, exactly: one key per
    sequence, so o = v_scale * e4m3(v) (each code is exact in 16 bits) and,
    with one-hot queries, lse = scale * k_scale * e4m3(k) of one column.  NaN
    codes (S.1111.111) give NaN where the oracle's arithmetic does: a NaN in
    V only in its column, a NaN anywhere in a key row in every head's score."""
    say(f"case fp8 kv decode, every code, {dt}")
    B, Hq, d = 16, 16, 128
    codes = np.arange(256, dtype=np.uint8)
    vc = np.stack([np.roll(codes, -d * b)[:d] for b in range(B)]).reshape(B, 1, 1, d)
    kc = np.zeros((B, 1, 1, d), np.uint8)
    for b in range(B):
        kc[b, 0, 0, :16] = codes[16 * b:16 * b + 16]     # head h reads column h
    q = torch.zeros((B, Hq, d), dtype=torch_dtype(dt))
    for h in range(Hq):
        q[:, h, h] = 1.0
    ks, vs, scale = 0.5, 1.0, 0.125
    o, lse, op, lp = attn().attn_decode_fp8kv(q.to(DEV), torch.from_numpy(kc).to(DEV), torch.from_numpy(vc).to(DEV),
                                              ks, vs, 128, scale)
    torch.cuda.synchronize()
    with np.errstate(invalid="ignore"):
        Or, Lr, _, _ = oracle.decode_fp8kv_ref(q, kc, vc, ks, vs, scale, 128)
    O, L = f64(o), f64(lse)
    assert np.array_equal(np.isnan(O), np.isnan(Or)) and np.array_equal(np.isnan(L), np.isnan(Lr))
    assert np.isnan(Lr).sum() == 2 * Hq and np.isnan(Or).sum() == 2 * Hq * d + (B - 2) * Hq   # the pins above
    fin = ~np.isnan(Or)
    assert np.array_equal(O[fin], Or[fin])                # exact: e4m3 values are 16-bit values
    ok = ~np.isnan(Lr)
    assert np.max(np.abs(L[ok] - Lr[ok])) <= 1e-6 * np.max(np.abs(Lr[ok]))


# fused decode (partials and merge in one launch): segments of 128-key chunks
# merged by the last workgroup of each row
FUSED_SHAPES = [
    # B, Hq, Hkv, M, d, dtype
    (1, 8, 8, 512, 128, "f16"),        # small decode workload
    (2, 8, 8, 65536, 128, "f16"),      # long decode workload
    (8, 32, 8, 16384, 128, "bf16"),    # grouped-query decode workload
    (3, 16, 4, 4097, 64, "f16"),       # a one-key tail chunk
    (2, 24, 8, 777, 128, "bf16"),      # groups of 3 heads
    (1, 32, 1, 300, 128, "bf16"),      # a group split over two 16-head slices
    (2, 16, 4, 1000, 32, "bf16"),
    (64, 32, 32, 1000, 64, "f16"),     # more rows than the grid: one segment per row
    (1, 1, 1, 1, 128, "f16"),          # a single key
    (2, 16, 4, 1000, 256, "bf16"),     # head dim 256
    (1, 8, 8, 4097, 256, "f16"),
]


@pytest.mark.parametrize("shape", FUSED_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_decode_fused(shape):
    B, Hq, Hkv, M, d, dt = shape
    say(f"case fused decode {shape}")
    q, k, v = decode_inputs(B, Hq, Hkv, M, d, dt, seed=M + 3)
    scale = float(np.float32(d ** -0.5))
    o, lse = attn().attn_decode_fused(q.to(DEV), k.to(DEV), v.to(DEV), scale)
    torch.cuda.synchronize()
    Or, Lr, _, _ = oracle.decode_ref(q, k, v, scale, 128)
    eo, el = maxerr(f64(o), Or), maxerr(f64(lse), Lr)
    say(f"  o={eo:.3e} lse={el:.3e}")
    assert eo <= TOL_O[dt] and el <= TOL_LSE


def test_decode_fused_workspace_reuse_and_determinism():
    """One workspace serves calls of several sizes in a row (each completed
    call leaves its counters at zero); repeated calls give identical bits."""
    say("case fused decode workspace reuse")
    shapes = [(2, 8, 8, 20000, 128, "f16"), (1, 16, 2, 3000, 64, "bf16"), (2, 8, 8, 20000, 128, "f16")]
    need = max(attn().attn_decode_fused_workspace_bytes(B, Hq, Hkv, M, d) for B, Hq, Hkv, M, d, _ in shapes)
    ws = torch.zeros(need, dtype=torch.uint8, device=DEV)
    outs = []
    for i, (B, Hq, Hkv, M, d, dt) in enumerate(shapes):
        q, k, v = decode_inputs(B, Hq, Hkv, M, d, dt, seed=40 + (i % 2))
        scale = float(np.float32(d ** -0.5))
        o, lse = attn().attn_decode_fused(q.to(DEV), k.to(DEV), v.to(DEV), scale, workspace=ws)
        torch.cuda.synchronize()
        Or, Lr, _, _ = oracle.decode_ref(q, k, v, scale, 128)
        assert maxerr(f64(o), Or) <= TOL_O[dt] and maxerr(f64(lse), Lr) <= TOL_LSE, i
        outs.append((o, lse))
    assert torch.equal(outs[0][0], outs[2][0]) and torch.equal(outs[0][1], outs[2][1])
    n_cnt = 16 * 4  # the first 256 bytes hold the row counters of these shapes
    assert int(ws[:n_cnt].count_nonzero()) == 0, "counters not reset"


@pytest.mark.parametrize("C,d,dt", [(1, 128, "f16"), (3, 64, "bf16"), (600, 128, "f16"), (37, 64, "f16"),
                                    (3, 256, "bf16")])
def test_lse_merge_standalone(C, d, dt):
    say(f"case lse_merge C={C} d={d} {dt}")
    g = torch.Generator("cpu").manual_seed(C)
    op = torch.randn((2, 3, C, d), generator=g)
    lp = torch.randn((2, 3, C), generator=g) * 4.0
    o, lse = attn().lse_merge(op.to(DEV), lp.to(DEV), torch_dtype(dt))
    torch.cuda.synchronize()
    Or, Lr = oracle.lse_merge_ref(op, lp)
    assert maxerr(f64(o), Or) <= TOL_O[dt]
    assert maxerr(f64(lse), Lr) <= TOL_LSE


# (batch, head) counts that select every column width of the merge workgroup:
# 4*QW columns per workgroup, QW in {4, 8, 16, 32} (d = 128, 256), {4, 8, 16} (d = 64)
# and {4, 8} (d = 32)
@pytest.mark.parametrize("B,Hq,C,d,dt", [(4, 32, 50, 128, "bf16"), (8, 32, 7, 128, "f16"),
                                         (16, 32, 3, 128, "bf16"), (8, 32, 20, 64, "f16"),
                                         (16, 32, 5, 64, "bf16"), (3, 5, 130, 64, "bf16"),
                                         (2, 3, 40, 32, "f16"), (16, 32, 9, 32, "bf16"),
                                         (8, 32, 7, 256, "f16"), (4, 32, 9, 256, "bf16"),
                                         (2, 32, 11, 256, "f16"), (2, 3, 40, 256, "bf16")])
def test_lse_merge_column_widths(B, Hq, C, d, dt):
    say(f"case lse_merge B={B} Hq={Hq} C={C} d={d} {dt}")
    g = torch.Generator("cpu").manual_seed(B * 1000 + C)
    # partials in the range of attention outputs (|O_c| < 4, where rounding O to
    # bf16 stays within the bf16 bound); over 65536 outputs a unit normal would not
    op = torch.randn((B, Hq, C, d), generator=g) * 0.5
    lp = torch.randn((B, Hq, C), generator=g) * 4.0
    o, lse = attn().lse_merge(op.to(DEV), lp.to(DEV), torch_dtype(dt))
    torch.cuda.synchronize()
    Or, Lr = oracle.lse_merge_ref(op, lp)
    assert maxerr(f64(o), Or) <= TOL_O[dt]
    assert maxerr(f64(lse), Lr) <= TOL_LSE


def test_decode_matches_prefill_single_query():
    say("case decode vs attn_fwd(N=1)")
    B, Hq, Hkv, M, d = 2, 8, 2, 777, 128
    q, k, v = decode_inputs(B, Hq, Hkv, M, d, "f16", seed=9)
    scale = float(np.float32(d ** -0.5))
    Od, Ld, _, _ = gpu_decode(q, k, v, 128, scale)
    Of, Lf = gpu_fwd(q[:, None].contiguous(), k.transpose(1, 2).contiguous(), v.transpose(1, 2).contiguous(),
                     False, scale)
    assert maxerr(Od, Of[:, 0]) <= 2 * TOL_O["f16"]
    assert maxerr(Ld, Lf[:, :, 0]) <= 2 * TOL_LSE


def test_decode_deterministic_and_complete():
    say("case decode determinism / NaN-poisoned outputs")
    q, k, v = decode_inputs(1, 8, 8, 1000, 128, "f16", seed=3)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    C = math.ceil(1000 / 128)
    op = torch.full((1, 8, C, 128), float("nan"), device=DEV)
    lp = torch.full((1, 8, C), float("nan"), device=DEV)
    attn().attn_decode_splitkv(qd, kd, vd, o_part=op, lse_part=lp)
    o = torch.full((1, 8, 128), float("nan"), device=DEV, dtype=torch.float16)
    lse = torch.full((1, 8), float("nan"), device=DEV)
    attn().lse_merge(op, lp, o=o, lse=lse)
    o2, l2, _, _ = attn().attn_decode(qd, kd, vd)
    torch.cuda.synchronize()
    assert not torch.isnan(op).any() and not torch.isnan(o).any() and not torch.isnan(lse).any()
    assert torch.equal(o, o2) and torch.equal(lse, l2)
