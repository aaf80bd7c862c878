"""Benchmark of the attention hot path on one MI355X.

One step = one causal GQA bf16 prefill forward (B=4, Hq=32, Hkv=8,
N=M=4096, d=128) plus one split-KV decode (B=2, H=8, M=65536, d=128, fp16,
chunks of 128 keys: partials and LSE merge in one launch), all through the C
ABI, with inputs already resident in HBM.  The decode rotates between two
independent K/V sets (1.07 GB together) so the 256 MB last-level cache cannot
serve repeats.

Prints ONE JSON line.  ``value`` is the prefill throughput in TFLOP/s
(4*B*Hq*N*M*d, halved for the causal mask) over the prefill kernel's average
duration, measured with HIP events on the launch stream; the decode result is
reported in the ``decode`` object: GB/s of K+V+q+O over the step's one-launch
decode, with the two-launch path (chunk kernel + merge) and the chunk kernel
alone, timed after the steps, beside it; ``roofline_decode`` is the one-launch
decode kernel's roofline.  ``configs`` holds all five
workloads (tiny MHA and small decode as latencies, the MHA fp16 d=64 prefill
as TFLOP/s, the two headline workloads), each with the largest deviation from
the CPU oracle over its whole output (checked after the timed region).  The
``decode_gqa`` object reports a grouped-query decode (B=8, Hq=32, Hkv=8,
M=16384, d=128, bf16; K/V counted once per kv head; two launches and one), and ``decode_paged`` /
``decode_fp8kv`` / ``decode_paged_fp8kv`` the same workload's chunk kernel
through the paged-KV (two launches and one), FP8-KV and paged FP8-KV entry points.  ``cpu_baseline``
is the oracle timed on the host on the causal GQA prefill (all of it) and on
the long decode.

    python bench.py [--gpus 1] [--steps 20] [--warmup 10] [--prewarm-s 1.5] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import pathlib
import statistics
import sys
import time

ROOT = pathlib.Path(__file__).resolve().parent
sys.path.insert(0, str(ROOT))

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA (published)
PEAK_HBM_GBPS = 8000.0      # MI355X HBM3E (published)
PREFILL = "prefill_causal_gqa_bf16_d128"
DECODE = "long_decode_fp16_d128"
DECODE_GQA = "gqa_decode_bf16_d128"
CONFIGS = {"C1": "tiny_mha_fp16_d64", "C2": "small_decode_fp16_d128", "C3": "prefill_mha_fp16_d64",
           "C4": PREFILL, "C5": DECODE}
KERNEL_SOURCES = {
    "prefill": ["attention_attn_fwd_06_amd/csrc/prefill_fwd.hip",
                "attention_attn_fwd_06_amd/csrc/device_common.h",
                "attention_attn_fwd_06_amd/csrc/lds_stage.h",
                "attention_attn_fwd_06_amd/csrc/launch.h"],
    "decode": ["attention_attn_fwd_06_amd/csrc/decode.hip",
               "attention_attn_fwd_06_amd/csrc/device_common.h",
               "attention_attn_fwd_06_amd/csrc/lds_stage.h",
               "attention_attn_fwd_06_amd/csrc/launch.h"],
}


def source_hash(kind: str) -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES[kind]:
        h.update((ROOT / rel).read_bytes())
    return h.hexdigest()[:16]


def read_traffic(kind: str, workload: str, key: str = "hbm_bytes_per_launch"):
    """HBM bytes per launch (the summary line ``key``) from the committed
    rocprofv3 counter summary, or None when the summary is missing or was
    taken on a different kernel source."""
    p = ROOT / "profiles" / f"{kind}_{workload}_traffic.md"
    if not p.exists():
        return None
    vals = {}
    for line in p.read_text().splitlines():
        if ":" in line and line.startswith("- "):
            name, val = line[2:].split(":", 1)
            vals[name.strip()] = val.strip().strip("`")
    if vals.get("kernel_source_sha256") != source_hash(kind):
        return None
    try:
        return float(vals[key])
    except (KeyError, ValueError):
        return None


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def blas_threads() -> int:
    from threadpoolctl import threadpool_info
    return max([i.get("num_threads", 1) for i in threadpool_info()] or [1])


def maxerr(a, b) -> float:
    import numpy as np
    return float(np.max(np.abs(np.asarray(a, np.float64) - np.asarray(b, np.float64))))


def oracle_checks(attn, dev, timing: bool):
    """Each of the five workloads once more on the GPU (seed 0), compared with
    the oracle over its whole output; the oracle runs on the causal GQA
    prefill and the long decode are timed as the CPU baseline."""
    import torch

    import oracle
    from workloads import WORKLOADS, attn_flops, decode_bytes, make_inputs
    res, base = {}, {}
    for key, name in CONFIGS.items():
        w = WORKLOADS[name]
        q, k, v = make_inputs(w, 0)
        if w.kind == "prefill":
            o, lse = attn.attn_fwd(q.to(dev), k.to(dev), v.to(dev), causal=w.causal, scale=w.scale)
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            Or, Lr = oracle.attn_ref(q, k, v, w.scale, w.causal)
            dt = time.perf_counter() - t0
            if name == PREFILL:
                base["prefill"] = (attn_flops(w.B, w.Hq, w.N, w.M, w.d, w.causal) / dt / 1e12, dt)
        else:
            o, lse, _, _ = attn.attn_decode(q.to(dev), k.to(dev), v.to(dev), w.chunk, w.scale)
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            Or, Lr, _, _ = oracle.decode_ref(q, k, v, w.scale, w.chunk)
            dt = time.perf_counter() - t0
            if name == DECODE:
                base["decode"] = (decode_bytes(w.B, w.Hq, w.Hkv, w.M, w.d) / dt / 1e9, dt)
        res[key] = {"max_dO": maxerr(o.float().cpu().double().numpy(), Or),
                    "max_dlse": maxerr(lse.cpu().double().numpy(), Lr),
                    "tol_O": 8e-3 if w.dtype == "bf16" else 2e-3, "tol_lse": 1e-3}
        res[key]["within_tolerance"] = res[key]["max_dO"] <= res[key]["tol_O"] and \
            res[key]["max_dlse"] <= res[key]["tol_lse"]
    cpu = None
    if timing:
        threads = blas_threads()
        pw, dw = WORKLOADS[PREFILL], WORKLOADS[DECODE]
        cpu = {"value": base["prefill"][0], "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
               "cpu_model": cpu_model(), "host_cores_available": len(os.sched_getaffinity(0)),
               "sample": f"the whole {pw.name} workload ({pw.B * pw.Hq} (batch, head) problems, full "
                         f"{pw.N}x{pw.M} S and P each, float64 numpy), {base['prefill'][1]:.1f} s; FLOPs "
                         f"credited with the causal-halved count",
               "decode": {"value": base["decode"][0], "unit": "GB/s",
                          "sample": f"the whole {dw.name} workload ({dw.B * dw.Hq * dw.num_chunks} chunk "
                                    f"partials and their merge), {base['decode'][1]:.1f} s; bytes = K+V+q+O"}}
    return res, cpu


def gqa_decode_rate(attn, w, args, dev):
    """Grouped-query decode (K/V read once per kv head) on two alternating K/V
    sets, timed with HIP events on the launch stream: the one-launch decode
    (``value``), and chunk + merge in two launches beside it."""
    import torch
    from workloads import decode_bytes, make_inputs
    q, k0, v0 = (t.to(dev) for t in make_inputs(w, args.seed))
    _, k1, v1 = (t.to(dev) for t in make_inputs(w, args.seed + 1))
    kv = [(k0, v0), (k1, v1)]
    C = w.num_chunks
    o_part = torch.empty((w.B, w.Hq, C, w.d), dtype=torch.float32, device=dev)
    lse_part = torch.empty((w.B, w.Hq, C), dtype=torch.float32, device=dev)
    o = torch.empty((w.B, w.Hq, w.d), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((w.B, w.Hq), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()

    def step(i, ev=None):
        kk, vv = kv[i % 2]
        if ev: ev[0].record(stream)
        attn.attn_decode_splitkv(q, kk, vv, w.chunk, w.scale, o_part=o_part, lse_part=lse_part, stream=stream)
        if ev: ev[1].record(stream)
        attn.lse_merge(o_part, lse_part, o=o, lse=lse, stream=stream)
        if ev: ev[2].record(stream)

    _prewarm(step, args)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    for i in range(args.steps):
        step(i, events[i])
    torch.cuda.synchronize()
    c_ms = statistics.mean(e[0].elapsed_time(e[1]) for e in events)
    cm_ms = statistics.mean(e[0].elapsed_time(e[2]) for e in events)
    # the same decode in one launch (partials of 128-key chunk runs and their merge)
    ws = torch.zeros(attn.attn_decode_fused_workspace_bytes(w.B, w.Hq, w.Hkv, w.M, w.d), dtype=torch.uint8,
                     device=dev)
    f_ms = _time_chunk(lambda i: attn.attn_decode_fused(q, kv[i % 2][0], kv[i % 2][1], w.scale, o=o, lse=lse,
                                                        workspace=ws), args)
    nbytes = decode_bytes(w.B, w.Hq, w.Hkv, w.M, w.d)
    chunk_bytes = nbytes - w.B * w.Hq * w.d * 2
    gbps = nbytes / (cm_ms * 1e-3) / 1e9
    f_gbps = nbytes / (f_ms * 1e-3) / 1e9
    return {"workload": w.desc, "value": round(f_gbps, 1), "unit": "GB/s", "frac": round(f_gbps / PEAK_HBM_GBPS, 4),
            "path": "attn_decode_fused (one launch)",
            "chunk_merge_GBps": round(gbps, 1), "chunk_merge_frac": round(gbps / PEAK_HBM_GBPS, 4),
            "chunk_merge_ms": round(cm_ms, 4), "chunk_ms": round(c_ms, 4),
            "chunk_only_GBps": round(chunk_bytes / (c_ms * 1e-3) / 1e9, 1),
            "fused_ms": round(f_ms, 4), "fused_GBps": round(f_gbps, 1), "fused_frac": round(f_gbps / PEAK_HBM_GBPS, 4),
            "kernel": "decode_gqa_mfma_kernel<128,bf16>", "algorithmic_bytes": nbytes,
            "bytes_note": "K and V counted once per kv head"}


def _prewarm(fn, args):
    """Untimed calls of fn(i) for up to half a second (at most --prewarm-s):
    each measurement starts after the input set-up on the host, an idle spell
    in which the GPU drops its clock, and the clock ramps up again only under
    load."""
    import torch
    t0 = time.perf_counter()
    i = 0
    while time.perf_counter() - t0 < min(0.5, args.prewarm_s):
        for _ in range(8):
            fn(i)
            i += 1
        torch.cuda.synchronize()


def _time_chunk(fn, args):
    """Mean HIP-event time (ms) of fn(i) on the current stream over args.steps
    calls, after the pre-warm and args.warmup untimed calls."""
    import torch
    stream = torch.cuda.current_stream()
    _prewarm(fn, args)
    for i in range(args.warmup):
        fn(i)
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    for i in range(args.steps):
        ev[i][0].record(stream)
        fn(i)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    return statistics.mean(a.elapsed_time(b) for a, b in ev)


def small_and_mha_rates(attn, args, dev):
    """The tiny MHA prefill and the small decode (latency-bound: microseconds
    per call, HIP events around each call) and the MHA fp16 d=64 prefill
    (TFLOP/s over its kernel time)."""
    import torch
    from workloads import WORKLOADS, attn_flops, make_inputs
    stream = torch.cuda.current_stream()
    out = {}
    w1 = WORKLOADS[CONFIGS["C1"]]
    q, k, v = (t.to(dev) for t in make_inputs(w1, args.seed))
    o, lse = torch.empty_like(q), torch.empty((w1.B, w1.Hq, w1.N), dtype=torch.float32, device=dev)
    us = 1e3 * _time_chunk(lambda i: attn.attn_fwd(q, k, v, causal=w1.causal, scale=w1.scale, o=o, lse=lse,
                                                    stream=stream), args)
    out["C1"] = {"workload": w1.desc, "us": round(us, 2), "kernel": "prefill_fwd_kernel<64,f16>"}
    w2 = WORKLOADS[CONFIGS["C2"]]
    q, k, v = (t.to(dev) for t in make_inputs(w2, args.seed))
    op = torch.empty((w2.B, w2.Hq, w2.num_chunks, w2.d), dtype=torch.float32, device=dev)
    lp = torch.empty((w2.B, w2.Hq, w2.num_chunks), dtype=torch.float32, device=dev)
    o2 = torch.empty((w2.B, w2.Hq, w2.d), dtype=torch.float16, device=dev)
    l2 = torch.empty((w2.B, w2.Hq), dtype=torch.float32, device=dev)

    def two_launches(i):
        attn.attn_decode_splitkv(q, k, v, w2.chunk, w2.scale, o_part=op, lse_part=lp, stream=stream)
        attn.lse_merge(op, lp, o=o2, lse=l2, stream=stream)
    us2 = 1e3 * _time_chunk(two_launches, args)
    ws = torch.zeros(attn.attn_decode_fused_workspace_bytes(w2.B, w2.Hq, w2.Hkv, w2.M, w2.d), dtype=torch.uint8,
                     device=dev)
    us2f = 1e3 * _time_chunk(lambda i: attn.attn_decode_fused(q, k, v, w2.scale, o=o2, lse=l2, workspace=ws,
                                                              stream=stream), args)
    out["C2"] = {"workload": w2.desc, "us_chunk_merge": round(us2, 2), "us_fused": round(us2f, 2)}
    w3 = WORKLOADS[CONFIGS["C3"]]
    q, k, v = (t.to(dev) for t in make_inputs(w3, args.seed))
    o3 = torch.empty_like(q)
    l3 = torch.empty((w3.B, w3.Hq, w3.N), dtype=torch.float32, device=dev)
    ms3 = _time_chunk(lambda i: attn.attn_fwd(q, k, v, causal=w3.causal, scale=w3.scale, o=o3, lse=l3,
                                               stream=stream), args)
    tf3 = attn_flops(w3.B, w3.Hq, w3.N, w3.M, w3.d, w3.causal) / (ms3 * 1e-3) / 1e12
    out["C3"] = {"workload": w3.desc, "ms": round(ms3, 4), "TFLOP/s": round(tf3, 2),
                 "frac": round(tf3 / PEAK_BF16_TFLOPS, 4), "kernel": "prefill_fwd_kernel<64,f16>",
                 "peak_note": "dense fp16 MFMA peak 2.5 PFLOP/s"}
    return out


def fp8qk_rate(attn, args, dev):
    """The causal GQA d=128 workload with Q and K as FP8 E4M3 codes (bf16 V):
    TFLOP/s over the kernel time.  Half of the FLOPs (Q K^T) run on the FP8
    matrix cores (5.0 PFLOP/s dense), half (P V) on the bf16 ones (2.5), so the
    peak for this mix is 1 / (0.5 / 5.0 + 0.5 / 2.5) = 3.33 PFLOP/s."""
    import torch
    from workloads import WORKLOADS, attn_flops, prefill_fp8qk_inputs
    w = WORKLOADS[PREFILL]
    q8, k8, v, qs, ks = (t.to(dev) if hasattr(t, "to") else t for t in
                         prefill_fp8qk_inputs(w.B, w.Hq, w.Hkv, w.N, w.M, w.d, "bf16", args.seed))
    o = torch.empty((w.B, w.N, w.Hq, w.d), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((w.B, w.Hq, w.N), dtype=torch.float32, device=dev)
    ms = _time_chunk(lambda i: attn.attn_fwd_fp8qk(q8, k8, v, qs, ks, causal=True, scale=w.scale, o=o, lse=lse), args)
    tf = attn_flops(w.B, w.Hq, w.N, w.M, w.d, w.causal) / (ms * 1e-3) / 1e12
    mixed_peak = 1.0 / (0.5 / 5000.0 + 0.5 / PEAK_BF16_TFLOPS)
    return {"workload": w.desc.replace("bf16", "FP8 E4M3 Q/K, bf16 V"), "ms": round(ms, 4), "TFLOP/s": round(tf, 2),
            "frac_of_bf16_peak": round(tf / PEAK_BF16_TFLOPS, 4), "frac_of_mixed_peak": round(tf / mixed_peak, 4),
            "kernel": "prefill_fwd_kernel<128,bf16,causal,fp8qk>"}


def paged_and_fp8_rates(attn, w, args, dev):
    """The grouped-query decode workload through the paged-KV entry points (block
    16, token-major pages in shuffled order, every sequence full length) and the
    FP8-KV ones (E4M3 codes): the one-launch decode (``value``) and the chunk
    kernel alone, two input sets alternated.  Bytes: K and V once per kv head
    (1 byte per element for FP8)."""
    import torch
    g = torch.Generator(device="cpu").manual_seed(args.seed)
    q = torch.randn((w.B, w.Hq, w.d), generator=g).to(torch.bfloat16).to(dev)
    C = w.num_chunks
    o_part = torch.empty((w.B, w.Hq, C, w.d), dtype=torch.float32, device=dev)
    lse_part = torch.empty((w.B, w.Hq, C), dtype=torch.float32, device=dev)
    out = {}
    bs = 16
    nb = w.B * w.M // bs
    sets = []
    for _ in range(2):
        kc = torch.randn((nb, bs, w.Hkv, w.d), dtype=torch.bfloat16, device=dev)
        vc = torch.randn((nb, bs, w.Hkv, w.d), dtype=torch.bfloat16, device=dev)
        table = torch.randperm(nb, generator=g).to(torch.int32).reshape(w.B, w.M // bs).to(dev)
        sets.append((kc, vc, table))
    lens = torch.full((w.B,), w.M, dtype=torch.int32, device=dev)
    ms = _time_chunk(lambda i: attn.attn_decode_paged_splitkv(q, sets[i % 2][0], sets[i % 2][1], sets[i % 2][2], lens,
                                                              w.chunk, w.scale, o_part=o_part, lse_part=lse_part), args)
    nbytes = 2.0 * w.B * w.Hkv * w.M * w.d * 2 + w.B * w.Hq * w.d * 2
    # the same paged decode in one launch (partials and merge fused)
    ws = torch.zeros(attn.attn_decode_fused_workspace_bytes(w.B, w.Hq, w.Hkv, w.M, w.d), dtype=torch.uint8,
                     device=dev)
    o = torch.empty((w.B, w.Hq, w.d), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((w.B, w.Hq), dtype=torch.float32, device=dev)
    ms_f = _time_chunk(lambda i: attn.attn_decode_paged_fused(q, sets[i % 2][0], sets[i % 2][1], sets[i % 2][2], lens,
                                                              w.scale, o=o, lse=lse, workspace=ws), args)
    out["decode_paged"] = {"workload": w.desc + ", paged KV: 16-key token-major pages, shuffled",
                           "value": round(nbytes / (ms_f * 1e-3) / 1e9, 1), "unit": "GB/s",
                           "frac": round(nbytes / (ms_f * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4),
                           "path": "attn_decode_paged_fused (one launch)", "fused_ms": round(ms_f, 4),
                           "chunk_ms": round(ms, 4), "chunk_only_GBps": round(nbytes / (ms * 1e-3) / 1e9, 1),
                           "chunk_only_frac": round(nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4),
                           "kernel": "decode_gqa_mfma_kernel<128,bf16,paged>"}
    del sets
    sets8 = [(torch.randint(0, 126, (w.B, w.Hkv, w.M, w.d), dtype=torch.uint8, device=dev),
              torch.randint(0, 126, (w.B, w.Hkv, w.M, w.d), dtype=torch.uint8, device=dev)) for _ in range(2)]
    ms8 = _time_chunk(lambda i: attn.attn_decode_fp8kv_splitkv(q, sets8[i % 2][0], sets8[i % 2][1], 0.01, 0.01,
                                                               w.chunk, w.scale, o_part=o_part, lse_part=lse_part),
                      args)
    nbytes8 = 2.0 * w.B * w.Hkv * w.M * w.d + w.B * w.Hq * w.d * 2
    # the same FP8-KV decode in one launch (partials and merge fused)
    ms8_f = _time_chunk(lambda i: attn.attn_decode_fp8kv_fused(q, sets8[i % 2][0], sets8[i % 2][1], 0.01, 0.01,
                                                               w.scale, o=o, lse=lse, workspace=ws), args)
    out["decode_fp8kv"] = {"workload": w.desc + ", K/V as FP8 E4M3 codes",
                           "value": round(nbytes8 / (ms8_f * 1e-3) / 1e9, 1), "unit": "GB/s",
                           "frac": round(nbytes8 / (ms8_f * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4),
                           "path": "attn_decode_fp8kv_fused (one launch)", "fused_ms": round(ms8_f, 4),
                           "chunk_ms": round(ms8, 4), "chunk_only_GBps": round(nbytes8 / (ms8 * 1e-3) / 1e9, 1),
                           "chunk_only_frac": round(nbytes8 / (ms8 * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4),
                           "kernel": "decode_gqa_mfma_kernel<128,bf16,fp8kv>"}
    del sets8
    sets8p = []
    for _ in range(2):
        kc = torch.randint(0, 126, (nb, bs, w.Hkv, w.d), dtype=torch.uint8, device=dev)
        vc = torch.randint(0, 126, (nb, bs, w.Hkv, w.d), dtype=torch.uint8, device=dev)
        table = torch.randperm(nb, generator=g).to(torch.int32).reshape(w.B, w.M // bs).to(dev)
        sets8p.append((kc, vc, table))
    ms8p = _time_chunk(lambda i: attn.attn_decode_paged_splitkv(q, sets8p[i % 2][0], sets8p[i % 2][1], sets8p[i % 2][2],
                                                                lens, w.chunk, w.scale, o_part=o_part,
                                                                lse_part=lse_part, k_scale=0.01, v_scale=0.01), args)
    ms8p_f = _time_chunk(lambda i: attn.attn_decode_paged_fused(q, sets8p[i % 2][0], sets8p[i % 2][1],
                                                                sets8p[i % 2][2], lens, w.scale, o=o, lse=lse,
                                                                workspace=ws, k_scale=0.01, v_scale=0.01), args)
    out["decode_paged_fp8kv"] = {"workload": w.desc + ", paged FP8 KV: 16-key token-major pages, shuffled",
                                 "value": round(nbytes8 / (ms8p_f * 1e-3) / 1e9, 1), "unit": "GB/s",
                                 "frac": round(nbytes8 / (ms8p_f * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4),
                                 "path": "attn_decode_paged_fused with FP8 caches (one launch)",
                                 "fused_ms": round(ms8p_f, 4), "chunk_ms": round(ms8p, 4),
                                 "chunk_only_GBps": round(nbytes8 / (ms8p * 1e-3) / 1e9, 1),
                                 "chunk_only_frac": round(nbytes8 / (ms8p * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4),
                                 "kernel": "decode_gqa_mfma_kernel<128,bf16,paged,fp8kv>"}
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--prewarm-s", type=float, default=1.5,
                    help="seconds of untimed steps before the counted warm-up (clock ramp)")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-oracle", action="store_true", help="skip the oracle checks and the CPU baseline")
    ap.add_argument("--only", choices=["prefill", "prefill_mha", "decode", "decode_fused", "decode_gqa", "copy"],
                    default=None, help="run one part only (for counter collection)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: this build measures one GPU only (got --gpus {args.gpus}); "
              "multi-GPU sharding is described in the design notes, not run", file=sys.stderr)
        sys.exit(2)

    import torch
    import attention_attn_fwd_06_amd as attn
    from workloads import WORKLOADS, attn_flops, decode_bytes, make_inputs

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    wp, wd = WORKLOADS[PREFILL], WORKLOADS[DECODE]

    if args.only == "copy":
        # Reference copy of a known size for scaling the HBM byte counters.
        n = 1 << 28  # 2^28 fp32 = 1 GiB read + 1 GiB written
        a = torch.empty(n, dtype=torch.float32, device=dev).uniform_()
        b = torch.empty_like(a)
        for _ in range(args.warmup + args.steps):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": n * 4, "copy_bytes_written": n * 4}))
        return

    if args.only == "prefill_mha":
        # the MHA fp16 d=64 prefill alone (for counter collection)
        w3 = WORKLOADS[CONFIGS["C3"]]
        q, k, v = (t.to(dev) for t in make_inputs(w3, args.seed))
        o3 = torch.empty_like(q)
        ms3 = _time_chunk(lambda i: attn.attn_fwd(q, k, v, causal=w3.causal, scale=w3.scale, o=o3), args)
        tf3 = attn_flops(w3.B, w3.Hq, w3.N, w3.M, w3.d, w3.causal) / (ms3 * 1e-3) / 1e12
        print(json.dumps({"workload": w3.desc, "ms": round(ms3, 4), "TFLOP/s": round(tf3, 2)}), flush=True)
        return
    if args.only == "decode_fused":
        # the fused long decode alone (for counter collection)
        q, k0, v0 = (t.to(dev) for t in make_inputs(wd, args.seed))
        _, k1, v1 = (t.to(dev) for t in make_inputs(wd, args.seed + 1))
        ws = torch.zeros(attn.attn_decode_fused_workspace_bytes(wd.B, wd.Hq, wd.Hkv, wd.M, wd.d), dtype=torch.uint8,
                         device=dev)
        kv = [(k0, v0), (k1, v1)]
        ms = _time_chunk(lambda i: attn.attn_decode_fused(q, kv[i % 2][0], kv[i % 2][1], wd.scale, workspace=ws), args)
        print(json.dumps({"workload": wd.desc, "ms": round(ms, 4)}), flush=True)
        return

    do_p = args.only in (None, "prefill")
    do_d = args.only in (None, "decode")
    if do_p:
        q, k, v = (t.to(dev) for t in make_inputs(wp, args.seed))
        o = torch.empty_like(q)
        lse = torch.empty((wp.B, wp.Hq, wp.N), dtype=torch.float32, device=dev)
    if do_d:
        dq, dk0, dv0 = (t.to(dev) for t in make_inputs(wd, args.seed))
        _, dk1, dv1 = (t.to(dev) for t in make_inputs(wd, args.seed + 1))
        kv_sets = [(dk0, dv0), (dk1, dv1)]
        C = wd.num_chunks
        o_part = torch.empty((wd.B, wd.Hq, C, wd.d), dtype=torch.float32, device=dev)
        lse_part = torch.empty((wd.B, wd.Hq, C), dtype=torch.float32, device=dev)
        do_ = torch.empty((wd.B, wd.Hq, wd.d), dtype=torch.float16, device=dev)
        dlse = torch.empty((wd.B, wd.Hq), dtype=torch.float32, device=dev)
        dws = torch.zeros(attn.attn_decode_fused_workspace_bytes(wd.B, wd.Hq, wd.Hkv, wd.M, wd.d),
                          dtype=torch.uint8, device=dev)

    stream = torch.cuda.current_stream()

    def step(i, ev=None):
        if do_p:
            if ev: ev[0].record(stream)
            attn.attn_fwd(q, k, v, causal=True, scale=wp.scale, o=o, lse=lse, stream=stream)
            if ev: ev[1].record(stream)
        if do_d:
            # the decode in one launch: chunk partials and their merge
            kk, vv = kv_sets[i % 2]
            if ev: ev[2].record(stream)
            attn.attn_decode_fused(dq, kk, vv, wd.scale, o=do_, lse=dlse, workspace=dws, stream=stream)
            if ev: ev[3].record(stream)

    def chunk_merge(i):
        # the two-launch path; no event between the launches (one there adds
        # about 3 us of its own)
        kk, vv = kv_sets[i % 2]
        attn.attn_decode_splitkv(dq, kk, vv, wd.chunk, wd.scale, o_part=o_part, lse_part=lse_part,
                                 stream=stream)
        attn.lse_merge(o_part, lse_part, o=do_, lse=dlse, stream=stream)

    def chunk_only(i):
        kk, vv = kv_sets[i % 2]
        attn.attn_decode_splitkv(dq, kk, vv, wd.chunk, wd.scale, o_part=o_part, lse_part=lse_part,
                                 stream=stream)

    # The GPU reaches its sustained clock only after about a second of load:
    # run untimed steps for --prewarm-s seconds, then the counted warm-up.
    t_pre = time.perf_counter()
    i = 0
    while time.perf_counter() - t_pre < args.prewarm_s:
        step(i)
        torch.cuda.synchronize()
        i += 1
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i, events[i])
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / args.steps
    if do_d:
        # the same decode in two launches (chunk kernel + merge), and the chunk
        # kernel alone, timed after the steps
        cm_ms = _time_chunk(chunk_merge, args)
        c_ms = _time_chunk(chunk_only, args)

    out = {
        "metric": "attn fwd TFLOP/s & % MFMA peak (prefill); decode HBM GB/s & % peak",
        "value": None, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(wall_ms, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"{PREFILL} + {DECODE}",
                   "prefill": wp.desc, "decode": wd.desc, "parallelism": "single GPU"},
    }
    if do_p:
        p_ms = statistics.mean(e[0].elapsed_time(e[1]) for e in events)
        flops = attn_flops(wp.B, wp.Hq, wp.N, wp.M, wp.d, wp.causal)
        tf = flops / (p_ms * 1e-3) / 1e12
        traffic = read_traffic("prefill", PREFILL)
        out["value"] = round(tf, 2)
        out["prefill_ms"] = round(p_ms, 4)
        out["roofline"] = {"bound": "mfma", "achieved": round(tf, 2), "peak": PEAK_BF16_TFLOPS,
                           "unit": "TFLOP/s", "frac": round(tf / PEAK_BF16_TFLOPS, 4),
                           "traffic": traffic, "kernel": "prefill_fwd_kernel<128,bf16,causal>",
                           "per_launch": f"{flops:.6g} FLOP (causal-halved)"}
    if do_d:
        f_ms = statistics.mean(e[2].elapsed_time(e[3]) for e in events)
        nbytes = decode_bytes(wd.B, wd.Hq, wd.Hkv, wd.M, wd.d)
        chunk_bytes = nbytes - wd.B * wd.Hq * wd.d * 2  # K+V+q (O is written by the merge)
        gbps = nbytes / (cm_ms * 1e-3) / 1e9
        f_gbps = nbytes / (f_ms * 1e-3) / 1e9
        # the step's decode is the one-launch path (attn_decode_fused); the
        # two-launch path (attn_decode_splitkv + lse_merge) is reported beside it
        out["decode"] = {"value": round(f_gbps, 1), "unit": "GB/s", "frac": round(f_gbps / PEAK_HBM_GBPS, 4),
                         "dtype": "f16", "ms": round(f_ms, 4), "path": "attn_decode_fused (one launch)",
                         "chunk_merge_ms": round(cm_ms, 4), "chunk_merge_GBps": round(gbps, 1),
                         "chunk_merge_frac": round(gbps / PEAK_HBM_GBPS, 4), "chunk_ms": round(c_ms, 4),
                         "chunk_only_GBps": round(chunk_bytes / (c_ms * 1e-3) / 1e9, 1),
                         "algorithmic_bytes": nbytes}
        out["roofline_decode"] = {"bound": "hbm", "achieved": round(f_gbps, 1),
                                  "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                                  "frac": round(f_gbps / PEAK_HBM_GBPS, 4),
                                  "traffic": read_traffic("decode", DECODE, "fused_hbm_bytes_per_launch"),
                                  "kernel": "decode_gqa_mfma_kernel<128,f16,fused>",
                                  "per_launch": f"{nbytes:.6g} B (K+V+q read, O written)"}
        if not do_p:
            out["value"], out["unit"], out["dtype"] = out["decode"]["value"], "GB/s", "f16"
    if args.only in (None, "decode_gqa"):
        out["decode_gqa"] = gqa_decode_rate(attn, WORKLOADS[DECODE_GQA], args, dev)
        out.update(paged_and_fp8_rates(attn, WORKLOADS[DECODE_GQA], args, dev))
        if args.only == "decode_gqa":
            out["value"], out["unit"], out["dtype"] = out["decode_gqa"]["value"], "GB/s", "bf16"
    if args.only is None:
        cfg = small_and_mha_rates(attn, args, dev)
        out["prefill_fp8qk"] = fp8qk_rate(attn, args, dev)
        cfg["C4"] = {"workload": wp.desc, "ms": out["prefill_ms"], "TFLOP/s": out["value"],
                     "frac": out["roofline"]["frac"], "kernel": out["roofline"]["kernel"]}
        cfg["C5"] = {"workload": wd.desc, "ms": out["decode"]["ms"], "GB/s": out["decode"]["value"],
                     "frac": out["decode"]["frac"], "path": out["decode"]["path"],
                     "ms_chunk_merge": out["decode"]["chunk_merge_ms"],
                     "GB/s_chunk_merge": out["decode"]["chunk_merge_GBps"],
                     "frac_chunk_merge": out["decode"]["chunk_merge_frac"]}
        if not args.no_oracle:
            checks, cpu = oracle_checks(attn, dev, timing=not args.no_cpu_baseline)
            for key, r in checks.items():
                cfg[key].update(r)
            if cpu is not None:
                out["cpu_baseline"] = cpu
        out["configs"] = cfg
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
