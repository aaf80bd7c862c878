"""Plant plausible mistakes in copies of the oracle and check that the pins
catch every one of them (CPU only).  The mistakes are planted by editing the
oracle's source text, so the real oracle is never touched."""
import pathlib
import types

import numpy as np
import pytest

from tests import pins

SRC = (pathlib.Path(__file__).resolve().parents[1] / "oracle" / "attention.py").read_text()

MUTANTS = {
    # name: (original text, planted mistake)
    "gqa_interleaved_heads": ("kh = h // group", "kh = h % Hkv"),
    "causal_off_by_one": ("keys[None, :] > rows[:, None] + off", "keys[None, :] >= rows[:, None] + off"),
    "causal_upper_triangle": ("keys[None, :] > rows[:, None] + off", "keys[None, :] < rows[:, None] + off"),
    "causal_chunk_top_left": ("keys[None, :] > rows[:, None] + off", "keys[None, :] > rows[:, None]"),
    "causal_chunk_offset_sign": ("off = M - N if causal else 0", "off = N - M if causal else 0"),
    "scale_dropped": ("S = float(scale) * (Qbh @ Kbh.T)", "S = (Qbh @ Kbh.T)"),
    "scale_squared": ("S = float(scale) * (Qbh @ Kbh.T)", "S = float(scale) ** 2 * (Qbh @ Kbh.T)"),
    "pv_uses_keys": ("O[b, :, h, :] = P @ Vbh", "O[b, :, h, :] = P @ Kbh[:, :Vbh.shape[1]]"),
    "max_over_wrong_axis": ("m = np.max(S, axis=-1, keepdims=True)", "m = np.max(S, axis=0, keepdims=True)"),
    "lse_without_max": ("m_safe + np.log(np.where(empty, 1.0, l))", "np.log(np.where(empty, 1.0, l))"),
    "lse_log2": ("m_safe + np.log(np.where(empty, 1.0, l))", "m_safe + np.log2(np.where(empty, 1.0, l))"),
    "softmax_unnormalised": ("E / np.where(empty, 1.0, l)", "E"),
    "exp_sign_flipped": ("E = np.exp(S - m_safe)", "E = np.exp(m_safe - S)"),
    "decode_tail_chunk_dropped": ("C = -(-M // chunk)", "C = M // chunk"),
    "decode_partial_unnormalised": ("/ l_c   # O_c", "  # O_c"),
    "decode_lse_without_max": ("m_c + np.log(l_c)", "np.log(l_c)"),
    "decode_scale_dropped": ("s = float(scale) * (k[b, kh, lo:hi, :] @ q[b, h, :])",
                             "s = (k[b, kh, lo:hi, :] @ q[b, h, :])"),
    "merge_weights_unnormalised": ("np.exp(lse_part - np.where(empty, 0.0, g))", "np.exp(lse_part - mx_safe)"),
    "merge_lse_without_max": ("mx_safe + np.log(np.sum(", "np.log(np.sum("),
    "merge_empty_row_nan": ("empty = mx == -np.inf", "empty = np.zeros_like(mx, dtype=bool)"),
    "merge_nan_row_as_empty": ("empty = mx == -np.inf", "empty = ~np.isfinite(mx)"),
    "merge_plain_average": ("O = np.sum(w[..., None] * o_part, axis=-2)", "O = np.mean(o_part, axis=-2)"),
    "paged_row_shifted": ("pages, rows = bt[b, t // bs], t % bs", "pages, rows = bt[b, t // bs], (t + 1) % bs"),
    "paged_page_in_order": ("pages, rows = bt[b, t // bs], t % bs", "pages, rows = t // bs, t % bs"),
    "paged_ignores_length": ("t = np.arange(int(sl[b]))", "t = np.arange(bt.shape[1] * bs)"),
    "paged_empty_chunks_weighted": ("lse_part = np.full((B, Hq, C), -np.inf)", "lse_part = np.zeros((B, Hq, C))"),
    "e4m3_bias_8": ("np.exp2((e - 7).astype(np.float64))", "np.exp2((e - 8).astype(np.float64))"),
    "e4m3_subnormal_as_normal": ("(m / 8.0) * 2.0 ** -6", "(1.0 + m / 8.0) * 2.0 ** -7"),
    "e4m3_sign_dropped": ("sign = np.where(c & 0x80, -1.0, 1.0)", "sign = 1.0"),
    "fp8kv_k_scale_dropped": ("k = e4m3_decode(k_codes) * float(np.float32(k_scale))", "k = e4m3_decode(k_codes)"),
    "fp8kv_scales_swapped": ("v = e4m3_decode(v_codes) * float(np.float32(v_scale))",
                             "v = e4m3_decode(v_codes) * float(np.float32(k_scale))"),
    "fp8qk_q_scale_dropped": ("q = e4m3_decode(q_codes) * float(np.float32(q_scale))", "q = e4m3_decode(q_codes)"),
    "fp8qk_k_scale_squared": ("k = e4m3_decode(k_codes) * float(np.float32(k_scale))",
                              "k = e4m3_decode(k_codes) * float(np.float32(k_scale)) ** 2"),
    "fp8qk_causal_dropped": ("return attn_ref(q, k, v, scale, causal)\n", "return attn_ref(q, k, v, scale, False)\n"),
}


def _mutant(name):
    old, new = MUTANTS[name]
    assert SRC.count(old) >= 1, f"mutation site for {name} not found in the oracle"
    mod = types.ModuleType(f"oracle_mutant_{name}")
    mod.__dict__["np"] = np
    exec(compile(SRC.replace(old, new), f"<mutant {name}>", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name):
    bad = pins.failing_checks(_mutant(name))
    assert bad, f"no pin caught the planted mistake {name}"
