"""Seeded synthetic workloads for the attention forward and split-KV decode.

This module holds no attention arithmetic.  It names the five workloads
(shapes, dtypes, scale, chunk size), draws their inputs from a seeded CPU
generator, and states the throughput accounting that the benchmark reports.
Both the CPU oracle's tests and the GPU path's tests and benchmark take their
inputs from here, so the two sides always see bit-identical values.

Input recipe: ``torch.Generator('cpu').manual_seed(seed)``, then q, k, v are
drawn in that order with ``torch.randn(shape, dtype=float32)`` and rounded
(round-to-nearest-even) to fp16 or bf16 (inputs too large to draw on the host
quickly, the 2.1 GB key slices of one decode test, come from the GPU's seeded
generator instead, and the oracle reads copies of them).  The pages' workloads are
i.i.d. N(0, 1) inputs of these shapes ("Flash Decoding" page, section 7;
"fmha sm120" page, section 3 benchmark).

Layouts (physical, contiguous):
  prefill  q, o [B, N, Hq, d];  k, v [B, M, Hkv, d];  lse [B, Hq, N] fp32
  decode   q, o [B, Hq, d];     k, v [B, Hkv, M, d];  lse [B, Hq]   fp32
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch

__all__ = [
    "Workload", "WORKLOADS", "workload", "prefill_inputs", "decode_inputs",
    "make_inputs", "attn_flops", "decode_bytes", "torch_dtype", "prefill_ramp_inputs", "prefill_fp8qk_inputs",
    "e4m3_codes",
]


def torch_dtype(name: str) -> torch.dtype:
    return {"f16": torch.float16, "bf16": torch.bfloat16}[name]


@dataclass(frozen=True)
class Workload:
    name: str
    kind: str            # "prefill" or "decode"
    B: int
    Hq: int
    Hkv: int
    M: int               # number of keys / values
    d: int
    dtype: str           # "f16" or "bf16"
    N: int = 1           # number of queries (1 for decode)
    causal: bool = False
    chunk: int = 128     # decode chunk size (keys per partial)
    desc: str = field(default="", compare=False)

    @property
    def scale(self) -> float:
        """1/sqrt(d) rounded to fp32: the value both sides receive."""
        return float(np.float32(1.0 / math.sqrt(self.d)))

    @property
    def num_chunks(self) -> int:
        return -(-self.M // self.chunk)


WORKLOADS = {
    w.name: w for w in [
        Workload("tiny_mha_fp16_d64", "prefill", B=1, Hq=2, Hkv=2, N=128, M=128, d=64,
                 dtype="f16", desc="tiny non-causal MHA, B=1 H=2 N=M=128 d=64 fp16"),
        Workload("small_decode_fp16_d128", "decode", B=1, Hq=8, Hkv=8, M=512, d=128,
                 dtype="f16", chunk=128,
                 desc="split-KV decode, B=1 H=8 M=512 d=128 fp16, 4 chunks of 128"),
        Workload("prefill_mha_fp16_d64", "prefill", B=16, Hq=16, Hkv=16, N=2048, M=2048, d=64,
                 dtype="f16", desc="non-causal MHA prefill, B=16 H=16 N=M=2048 d=64 fp16"),
        Workload("prefill_causal_gqa_bf16_d128", "prefill", B=4, Hq=32, Hkv=8, N=4096, M=4096,
                 d=128, dtype="bf16", causal=True,
                 desc="causal GQA prefill, B=4 Hq=32 Hkv=8 N=M=4096 d=128 bf16"),
        Workload("long_decode_fp16_d128", "decode", B=2, Hq=8, Hkv=8, M=65536, d=128,
                 dtype="f16", chunk=128,
                 desc="split-KV decode, B=2 H=8 M=65536 d=128 fp16, 512 chunks of 128"),
        Workload("gqa_decode_bf16_d128", "decode", B=8, Hq=32, Hkv=8, M=16384, d=128,
                 dtype="bf16", chunk=128,
                 desc="split-KV GQA decode, B=8 Hq=32 Hkv=8 M=16384 d=128 bf16, 128 chunks of 128"),
    ]
}


def workload(name: str) -> Workload:
    return WORKLOADS[name]


def _draw(shapes, dtype: str, seed: int, device: str = "cpu"):
    g = torch.Generator(device).manual_seed(seed)
    out = []
    for shape in shapes:
        x = torch.randn(shape, dtype=torch.float32, generator=g, device=device)
        out.append(x.to(torch_dtype(dtype)))
    return out


def prefill_inputs(B, Hq, Hkv, N, M, d, dtype="f16", seed=0):
    """q [B,N,Hq,d], k [B,M,Hkv,d], v [B,M,Hkv,d] on the CPU, rounded to ``dtype``."""
    return tuple(_draw([(B, N, Hq, d), (B, M, Hkv, d), (B, M, Hkv, d)], dtype, seed))


def decode_inputs(B, Hq, Hkv, M, d, dtype="f16", seed=0, device="cpu"):
    """q [B,Hq,d], k [B,Hkv,M,d], v [B,Hkv,M,d], rounded to ``dtype``; drawn on
    the CPU, or with the given device's generator (another stream of numbers,
    for inputs too large to draw on the host quickly)."""
    return tuple(_draw([(B, Hq, d), (B, Hkv, M, d), (B, Hkv, M, d)], dtype, seed, device))


def prefill_ramp_inputs(B, Hq, Hkv, N, M, d, dtype="f16", seed=0, a=4.0, slope=6.0, v_scale=0.25):
    """Prefill inputs whose scores grow with the key index, so that a row's
    maximum keeps rising from one block of keys to the next.

    With u = (1, ..., 1) / sqrt(d) (a unit vector) and i.i.d. N(0, 1) draws
    g_q, g_k, g_v (drawn in that order from the seeded generator):
        q[b, i, h]  = g_q + a * u
        k[b, j, kh] = g_k + slope * (j / 64) * u
        v           = v_scale * g_v
    so q.k_j carries a term a * slope * j / 64 that rises by a * slope per 64
    keys; v is scaled down so that |O| stays well below 2.  Rounded to
    ``dtype`` like the other inputs."""
    g = torch.Generator("cpu").manual_seed(seed)
    gq = torch.randn((B, N, Hq, d), dtype=torch.float32, generator=g)
    gk = torch.randn((B, M, Hkv, d), dtype=torch.float32, generator=g)
    gv = torch.randn((B, M, Hkv, d), dtype=torch.float32, generator=g)
    u = torch.full((d,), 1.0 / math.sqrt(d))
    ramp = (slope * torch.arange(M, dtype=torch.float32) / 64.0)[None, :, None, None]
    q = gq + a * u
    k = gk + ramp * u
    v = v_scale * gv
    return tuple(x.to(torch_dtype(dtype)) for x in (q, k, v))


def e4m3_codes(x: torch.Tensor):
    """Per-tensor quantisation to OCP FP8 E4M3 codes, as a caller would do it:
    scale = max|x| / 448 (rounded to fp32), codes = round-to-nearest-even of
    x / scale in E4M3 (torch's float8_e4m3fn conversion), as uint8.  Returns
    (codes, scale)."""
    scale = float(np.float32(float(x.abs().max()) / 448.0)) or 1.0
    codes = (x.float() / scale).clamp(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8)
    return codes, scale


def prefill_fp8qk_inputs(B, Hq, Hkv, N, M, d, dtype="bf16", seed=0):
    """q, k, v drawn as ``prefill_inputs`` (float32 before rounding); q and k
    quantised to E4M3 codes with per-tensor scales (``e4m3_codes``), v rounded
    to ``dtype``.  Returns (q8, k8, v, q_scale, k_scale)."""
    g = torch.Generator("cpu").manual_seed(seed)
    q = torch.randn((B, N, Hq, d), dtype=torch.float32, generator=g)
    k = torch.randn((B, M, Hkv, d), dtype=torch.float32, generator=g)
    v = torch.randn((B, M, Hkv, d), dtype=torch.float32, generator=g)
    q8, qs = e4m3_codes(q)
    k8, ks = e4m3_codes(k)
    return q8, k8, v.to(torch_dtype(dtype)), qs, ks


def make_inputs(w: Workload, seed: int = 0):
    if w.kind == "prefill":
        return prefill_inputs(w.B, w.Hq, w.Hkv, w.N, w.M, w.d, w.dtype, seed)
    return decode_inputs(w.B, w.Hq, w.Hkv, w.M, w.d, w.dtype, seed)


# ----------------------------------------------------------------------------
# Throughput accounting ("fmha sm120" page, section 3 benchmark table;
# "Flash Decoding" page, sections 7.1-7.2 roofline).
# ----------------------------------------------------------------------------

def attn_flops(B, Hq, N, M, d, causal) -> float:
    """Algorithmic FLOPs of the forward: two N x M x d products, 2 FLOP per MAC,
    halved under the causal mask.  Softmax work and masked-tile waste are not
    counted, matching the benchmark table of the "fmha sm120" page."""
    f = 4.0 * B * Hq * N * M * d
    return f / 2.0 if causal else f


def decode_bytes(B, Hq, Hkv, M, d, elem_bytes=2) -> float:
    """Algorithmic HBM bytes of one decode step: K and V read once, q read and
    O written once (the page's roofline counts the K/V stream)."""
    kv = 2.0 * B * Hkv * M * d * elem_bytes
    qo = 2.0 * B * Hq * d * elem_bytes
    return kv + qo
