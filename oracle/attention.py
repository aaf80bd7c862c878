"""Plain float64 definitions of what the fused attention path computes.

TEST INFRASTRUCTURE: imported only by the tests, the smoke entry point and the
benchmark's CPU-baseline leg; never by the product path.

Sources (pages and their sections):
  * "fmha sm120: beyond torch.sdpa" (WingEdge777), section 1 "flash attention":
    multi-head attention is s = q.k^T * scale, p = softmax(s), o = p.v, with
    q, k, v laid out [batch, seq, heads, head_dim]; section 2 "fmha
    implementation": grouped-query heads use kv_head = q_head // (Hq / Hkv),
    and the causal mask keeps key j for query i when i >= j (top-left).
  * "CUDA Flash Decoding" (yunpan.plus), section 2.2 "chunk partial + global
    LSE weighted reduce": per chunk c, S_c = q.K_c^T, m_c = max S_c,
    P_c = exp(S_c - m_c), l_c = sum P_c, O_c = P_c.V_c / l_c,
    lse_c = m_c + log l_c; then global_lse = log sum_c exp(lse_c),
    w_c = exp(lse_c - global_lse), O = sum_c w_c O_c.
  * "Tensor Core migration plan" (CuFlash-Attn design doc), cross-cutting
    notes: the log-sum-exp row statistic is kept as fp32 output.

Readings where the pages leave a step open (each is also listed in the design
notes of the repository):
  * lse is the natural logarithm of the row's softmax denominator including
    the max: lse_i = m_i + ln(l_i) = ln sum_j exp(S_ij).
  * The causal mask for N <= M keys key j for query i when j <= i + (M - N):
    the queries are the last N positions of the key sequence (a chunk of a
    longer prefill), so the last query sees every key.  For N == M this is
    the pages' top-left mask; N > M is not defined here.  The reading makes a
    chunk's rows equal the same rows of the full-length causal attention.
  * A row with no allowed key has O = 0 and lse = -inf (unreachable with
    this mask and N <= M, since key 0 is always allowed).
  * Inputs are the already-rounded fp16/bf16 values upcast exactly to
    float64; ``scale`` is the fp32 value handed to the GPU, upcast.
  * Paged KV (the pages name it only as future work, with no layout): pages
    of block_size consecutive keys of every KV head, [num_blocks, block_size,
    Hkv, d]; key t of sequence b is row t % block_size of page
    block_table[b, t // block_size]; sequence b holds seq_lens[b] keys.  A
    paged decode computes exactly the decode of each sequence's gathered keys;
    chunks past a sequence's end have O_c = 0 and lse_c = -inf (no weight in
    the merge).
  * FP8 KV (the "fmha sm120" page lists fp8 KV quantisation as future work,
    with no format): K and V are OCP FP8 E4M3 codes with one fp32 scale each,
    K = k_scale * e4m3(k), V = v_scale * e4m3(v); the decode of these values is
    the plain decode.  E4M3 (OCP "e4m3fn"): sign bit, 4 exponent bits with bias
    7, 3 mantissa bits; exponent 0 is subnormal (m/8 * 2^-6); S.1111.111 is NaN;
    there are no infinities.
  * FP8 attention (the same TODO item; no format on the pages): Q and K given
    as E4M3 codes with one fp32 scale each, Q = q_scale * e4m3(q),
    K = k_scale * e4m3(k), V in 16 bits; the result is the plain attention of
    these values (the kernel's products of E4M3 values are exact).
"""
from __future__ import annotations

import numpy as np

__all__ = ["attn_ref", "decode_partials_ref", "lse_merge_ref", "decode_ref", "paged_decode_partials_ref",
           "paged_decode_ref", "e4m3_decode", "decode_fp8kv_partials_ref", "decode_fp8kv_ref", "attn_fp8qk_ref"]


def _f64(x) -> np.ndarray:
    """Exact upcast of a torch tensor or numpy array to float64."""
    if hasattr(x, "detach"):  # torch tensor (fp16/bf16/fp32 upcast is exact)
        x = x.detach().to("cpu").double().numpy()
    return np.asarray(x, dtype=np.float64)


def _softmax_rows(S: np.ndarray):
    """Row softmax of a score matrix whose disallowed entries are -inf.

    Returns (P, lse) with P normalised along the last axis and
    lse = m + ln(sum exp(S - m)), the natural-log row log-sum-exp.
    Rows with no finite entry give P = 0 and lse = -inf.
    """
    m = np.max(S, axis=-1, keepdims=True)
    empty = ~np.isfinite(m)
    m_safe = np.where(empty, 0.0, m)
    E = np.exp(S - m_safe)                 # exp(-inf) = 0 for masked keys
    l = np.sum(E, axis=-1, keepdims=True)
    P = np.where(empty, 0.0, E / np.where(empty, 1.0, l))
    with np.errstate(divide="ignore"):
        lse = np.where(empty, -np.inf, m_safe + np.log(np.where(empty, 1.0, l)))
    return P, lse[..., 0]


def attn_ref(q, k, v, scale: float, causal: bool = False, rows=None):
    """Attention forward, materialising S and P per (batch, query head).

    q [B, N, Hq, d]; k [B, M, Hkv, d]; v [B, M, Hkv, dv] (the "fmha sm120"
    page's layout; the pages use dv = d).
    Returns O [B, n, Hq, dv] and lse [B, Hq, n] in float64, where n = N, or
    n = len(rows) when ``rows`` selects a subset of query positions (the
    causal mask still uses each row's absolute position; with causal, query
    i may see keys 0 .. i + M - N).
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, N, Hq, d = q.shape
    Bk, M, Hkv, dk = k.shape
    if (Bk, dk) != (B, d) or v.shape[:3] != k.shape[:3]:
        raise ValueError("shape mismatch between q, k, v")
    if Hq % Hkv != 0:
        raise ValueError("Hq must be a multiple of Hkv")
    if causal and N > M:
        raise ValueError("causal attention is defined here only for N <= M")
    off = M - N if causal else 0                  # query i sees keys j <= i + off
    group = Hq // Hkv
    rows = np.arange(N) if rows is None else np.asarray(rows, dtype=np.int64)
    n = rows.shape[0]

    O = np.zeros((B, n, Hq, v.shape[3]))
    lse = np.zeros((B, Hq, n))
    keys = np.arange(M)
    for b in range(B):
        for h in range(Hq):
            kh = h // group                       # contiguous query-head groups
            Qbh = q[b, rows, h, :]                # [n, d]
            Kbh = k[b, :, kh, :]                  # [M, d]
            Vbh = v[b, :, kh, :]                  # [M, dv]
            S = float(scale) * (Qbh @ Kbh.T)      # [n, M]
            if causal:
                S = np.where(keys[None, :] > rows[:, None] + off, -np.inf, S)
            P, lse_bh = _softmax_rows(S)
            O[b, :, h, :] = P @ Vbh
            lse[b, h, :] = lse_bh
    return O, lse


def decode_partials_ref(q, k, v, scale: float, chunk: int):
    """Per-chunk partials of single-query attention (Flash Decoding step 1).

    q [B, Hq, d]; k, v [B, Hkv, M, d] (the decode page's per-head KV layout).
    Chunk c covers keys [c*chunk, min((c+1)*chunk, M)); the last chunk may be
    shorter.  Returns o_part [B, Hq, C, d] (each chunk's *normalised* output)
    and lse_part [B, Hq, C] (m_c + ln l_c), C = ceil(M / chunk).
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, Hq, d = q.shape
    Bk, Hkv, M, dk = k.shape
    if (Bk, dk) != (B, d) or v.shape != k.shape:
        raise ValueError("shape mismatch between q, k, v")
    if Hq % Hkv != 0:
        raise ValueError("Hq must be a multiple of Hkv")
    group = Hq // Hkv
    C = -(-M // chunk)
    o_part = np.zeros((B, Hq, C, d))
    lse_part = np.zeros((B, Hq, C))
    for b in range(B):
        for h in range(Hq):
            kh = h // group
            for c in range(C):
                lo, hi = c * chunk, min((c + 1) * chunk, M)
                s = float(scale) * (k[b, kh, lo:hi, :] @ q[b, h, :])   # S_c [len]
                m_c = np.max(s)
                p = np.exp(s - m_c)                                   # P_c
                l_c = np.sum(p)                                       # l_c
                o_part[b, h, c, :] = (p @ v[b, kh, lo:hi, :]) / l_c   # O_c
                lse_part[b, h, c] = m_c + np.log(l_c)                 # lse_c
    return o_part, lse_part


def lse_merge_ref(o_part, lse_part):
    """Log-sum-exp weighted merge of chunk partials (Flash Decoding step 2).

    o_part [..., C, d], lse_part [..., C] -> O [..., d], lse [...]:
    g = max_c lse_c + ln sum_c exp(lse_c - max_c lse_c),
    w_c = exp(lse_c - g), O = sum_c w_c O_c, lse = g.
    A row whose chunks are all empty (every lse_c = -inf: no key at all) has
    no weight to spread: O = 0, lse = -inf, as for a row with no allowed key.
    """
    o_part, lse_part = _f64(o_part), _f64(lse_part)
    mx = np.max(lse_part, axis=-1, keepdims=True)
    empty = mx == -np.inf           # all partials -inf: no key (NaN partials stay NaN)
    mx_safe = np.where(empty, 0.0, mx)
    with np.errstate(divide="ignore"):
        g = np.where(empty, -np.inf, mx_safe + np.log(np.sum(np.exp(lse_part - mx_safe), axis=-1, keepdims=True)))
    w = np.where(empty, 0.0, np.exp(lse_part - np.where(empty, 0.0, g)))    # [..., C]
    O = np.sum(w[..., None] * o_part, axis=-2)
    return O, g[..., 0]


def decode_ref(q, k, v, scale: float, chunk: int):
    """Split-KV decode end to end: partials, then merge.  Returns
    (O [B, Hq, d], lse [B, Hq], o_part, lse_part)."""
    o_part, lse_part = decode_partials_ref(q, k, v, scale, chunk)
    O, lse = lse_merge_ref(o_part, lse_part)
    return O, lse, o_part, lse_part


def paged_decode_partials_ref(q, k_cache, v_cache, block_table, seq_lens, scale: float, chunk: int):
    """Split-KV decode partials over a paged KV cache (see the module notes for
    the page layout).

    q [B, Hq, d]; k_cache, v_cache [num_blocks, block_size, Hkv, d];
    block_table [B, max_blocks] page ids; seq_lens [B] key counts.  Returns
    o_part [B, Hq, C, d] and lse_part [B, Hq, C] with
    C = ceil(max_blocks * block_size / chunk): sequence b's chunks are those of
    ``decode_partials_ref`` on its gathered keys, the chunks past its end are
    O_c = 0, lse_c = -inf.
    """
    q, kc, vc = _f64(q), _f64(k_cache), _f64(v_cache)
    bt = np.asarray(block_table, dtype=np.int64)
    sl = np.asarray(seq_lens, dtype=np.int64)
    B, Hq, d = q.shape
    _, bs, Hkv, dk = kc.shape
    if dk != d or vc.shape != kc.shape or bt.shape[0] != B or sl.shape != (B,):
        raise ValueError("shape mismatch between q, the caches, block_table and seq_lens")
    C = -(-(bt.shape[1] * bs) // chunk)
    o_part = np.zeros((B, Hq, C, d))
    lse_part = np.full((B, Hq, C), -np.inf)
    for b in range(B):
        t = np.arange(int(sl[b]))                       # the sequence's keys
        pages, rows = bt[b, t // bs], t % bs
        kb = kc[pages, rows].transpose(1, 0, 2)[None]   # [1, Hkv, len, d]
        vb = vc[pages, rows].transpose(1, 0, 2)[None]
        op, lp = decode_partials_ref(q[b:b + 1], kb, vb, scale, chunk)
        o_part[b, :, :op.shape[2]] = op[0]
        lse_part[b, :, :lp.shape[2]] = lp[0]
    return o_part, lse_part


def paged_decode_ref(q, k_cache, v_cache, block_table, seq_lens, scale: float, chunk: int):
    """Paged split-KV decode end to end.  Returns (O [B, Hq, d], lse [B, Hq],
    o_part, lse_part)."""
    o_part, lse_part = paged_decode_partials_ref(q, k_cache, v_cache, block_table, seq_lens, scale, chunk)
    O, lse = lse_merge_ref(o_part, lse_part)
    return O, lse, o_part, lse_part


def e4m3_decode(codes):
    """Values of OCP FP8 E4M3 codes (uint8), from the format's definition."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    mag = np.where(e == 0, (m / 8.0) * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2((e - 7).astype(np.float64)))
    mag = np.where((e == 15) & (c & 0x7 == 7), np.nan, mag)
    return sign * mag


def decode_fp8kv_partials_ref(q, k_codes, v_codes, k_scale: float, v_scale: float, scale: float, chunk: int):
    """Split-KV decode partials with K/V given as E4M3 codes and fp32 scales:
    the decode of K = k_scale * e4m3(k), V = v_scale * e4m3(v)."""
    k = e4m3_decode(k_codes) * float(np.float32(k_scale))
    v = e4m3_decode(v_codes) * float(np.float32(v_scale))
    return decode_partials_ref(q, k, v, scale, chunk)


def decode_fp8kv_ref(q, k_codes, v_codes, k_scale: float, v_scale: float, scale: float, chunk: int):
    """FP8-KV split-KV decode end to end.  Returns (O, lse, o_part, lse_part)."""
    o_part, lse_part = decode_fp8kv_partials_ref(q, k_codes, v_codes, k_scale, v_scale, scale, chunk)
    O, lse = lse_merge_ref(o_part, lse_part)
    return O, lse, o_part, lse_part


def attn_fp8qk_ref(q_codes, k_codes, v, q_scale: float, k_scale: float, scale: float, causal: bool = False):
    """Attention with Q and K given as E4M3 codes and fp32 scales: the
    forward of Q = q_scale * e4m3(q_codes), K = k_scale * e4m3(k_codes) and V.
    Returns (O, lse) as ``attn_ref``."""
    q = e4m3_decode(q_codes) * float(np.float32(q_scale))
    k = e4m3_decode(k_codes) * float(np.float32(k_scale))
    return attn_ref(q, k, v, scale, causal)
