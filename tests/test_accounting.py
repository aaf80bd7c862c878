"""The benchmark's throughput accounting against the figures the pages print
(CPU only)."""
import pathlib

import pytest

from workloads import WORKLOADS, attn_flops, decode_bytes

GOLD = pathlib.Path(__file__).resolve().parent / "golden"


def _rows(name):
    for line in (GOLD / name).read_text().splitlines():
        if line.strip() and not line.startswith("#"):
            yield [float(x) for x in line.split()]


def test_causal_flops_reproduce_fmha_sm120_table():
    rows = list(_rows("fmha_sm120_causal_bf16_table.txt"))
    assert len(rows) == 5
    for B, H, d, n, ms, tflops in rows:
        f = attn_flops(int(B), int(H), int(n), int(n), int(d), causal=True)
        assert f / (ms * 1e-3) / 1e12 == pytest.approx(tflops, abs=0.006)


def test_decode_bytes_reproduce_flash_decoding_roofline():
    rows = list(_rows("flash_decoding_roofline.txt"))
    assert len(rows) == 2
    for B, H, M, d, mb, gbps, ms in rows:
        kv = decode_bytes(int(B), int(H), int(H), int(M), int(d)) - 2 * B * H * d * 2
        assert kv / 1e6 == pytest.approx(mb, abs=0.5)
        assert kv / (gbps * 1e9) * 1e3 == pytest.approx(ms, abs=0.006)


def test_workload_table():
    w = WORKLOADS["prefill_causal_gqa_bf16_d128"]
    assert attn_flops(w.B, w.Hq, w.N, w.M, w.d, w.causal) == pytest.approx(5.4976e11, rel=1e-4)
    w = WORKLOADS["prefill_mha_fp16_d64"]
    assert attn_flops(w.B, w.Hq, w.N, w.M, w.d, w.causal) == pytest.approx(2.7488e11, rel=1e-4)
    w = WORKLOADS["long_decode_fp16_d128"]
    assert w.num_chunks == 512
    assert decode_bytes(w.B, w.Hq, w.Hkv, w.M, w.d) == pytest.approx(5.3688e8, rel=1e-4)
    assert WORKLOADS["small_decode_fp16_d128"].num_chunks == 4
