"""Checks that pin the CPU oracle to something other than itself.

Every check takes the oracle as a parameter (a module exposing ``attn_ref``,
``decode_partials_ref``, ``lse_merge_ref``, ``decode_ref`` and the paged
variants) and raises
AssertionError when the oracle disagrees with:
  * a pure-Python brute force (``tests/brute.py``) on tiny inputs and on the
    whole of the two small workloads;
  * torch's float64 CPU ``scaled_dot_product_attention`` (a library routine
    that computes the same definition; its ``is_causal`` mask is top-left);
  * closed forms and invariants that the mathematics fixes.

The same checks run against the real oracle (all must pass) and against
copies of the oracle with a planted mistake (each must fail at least one),
which shows that the pins can see a dropped term, a wrong sign or index, or a
swapped operand.
"""
from __future__ import annotations

import math

import numpy as np
import torch

from tests.brute import brute_attention, brute_decode, brute_decode_partials

TOL = 1e-11


def _rand(shape, seed, scale=1.0):
    g = np.random.default_rng(seed)
    return g.standard_normal(shape) * scale


def _close(a, b, tol=TOL, what=""):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    err = np.max(np.abs(a - b)) if a.size else 0.0
    assert err <= tol, f"{what}: max abs diff {err:.3e} > {tol:.1e}"


# ---------------------------------------------------------------------------
# Brute force
# ---------------------------------------------------------------------------

PREFILL_TINY = [
    # B, N, M, Hq, Hkv, d, causal, scale
    (1, 5, 5, 2, 1, 3, False, 0.7),
    (1, 6, 6, 2, 2, 4, True, 0.5),
    (2, 7, 7, 4, 2, 5, True, 0.3),
    (2, 3, 9, 3, 1, 4, False, 1.1),
    (1, 1, 1, 1, 1, 2, True, 0.9),
    # causal with fewer queries than keys (the last N positions of the sequence)
    (1, 3, 8, 2, 1, 3, True, 0.8),
    (2, 1, 6, 2, 2, 4, True, 0.6),
]


def check_brute_prefill_tiny(ora):
    for i, (B, N, M, Hq, Hkv, d, causal, sc) in enumerate(PREFILL_TINY):
        q = _rand((B, N, Hq, d), 10 + i)
        k = _rand((B, M, Hkv, d), 20 + i)
        v = _rand((B, M, Hkv, d), 30 + i)
        O, lse = ora.attn_ref(q, k, v, sc, causal)
        Ob, Lb = brute_attention(q, k, v, sc, causal)
        _close(O, Ob, what=f"O case {i}")
        _close(lse, Lb, what=f"lse case {i}")


def check_brute_decode_tiny(ora):
    # a tail chunk (M not a multiple of chunk), GQA, chunk larger than M
    for i, (B, Hq, Hkv, M, d, chunk) in enumerate([(1, 2, 1, 10, 3, 4), (2, 4, 2, 7, 5, 3),
                                                   (1, 1, 1, 5, 4, 8)]):
        q = _rand((B, Hq, d), 40 + i)
        k = _rand((B, Hkv, M, d), 50 + i)
        v = _rand((B, Hkv, M, d), 60 + i)
        op, lp = ora.decode_partials_ref(q, k, v, 0.6, chunk)
        opb, lpb = brute_decode_partials(q, k, v, 0.6, chunk)
        _close(op, opb, what=f"o_part case {i}")
        _close(lp, lpb, what=f"lse_part case {i}")
        O, L, _, _ = ora.decode_ref(q, k, v, 0.6, chunk)
        Ob, Lb = brute_decode(q, k, v, 0.6)
        _close(O, Ob, what=f"merged O case {i}")
        _close(L, Lb, what=f"merged lse case {i}")


def check_brute_workload(ora, w, seed=0):
    """The whole of a small workload against brute force (a few seconds)."""
    from workloads import make_inputs
    q, k, v = make_inputs(w, seed)
    if w.kind == "prefill":
        O, lse = ora.attn_ref(q, k, v, w.scale, w.causal)
        Ob, Lb = brute_attention(q, k, v, w.scale, w.causal)
        _close(O, Ob, 1e-12, "O")
        _close(lse, Lb, 1e-12, "lse")
    else:
        O, L, op, lp = ora.decode_ref(q, k, v, w.scale, w.chunk)
        opb, lpb = brute_decode_partials(q, k, v, w.scale, w.chunk)
        Ob, Lb = brute_decode(q, k, v, w.scale)
        _close(op, opb, 1e-12, "o_part")
        _close(lp, lpb, 1e-12, "lse_part")
        _close(O, Ob, 1e-12, "O")
        _close(L, Lb, 1e-12, "lse")


# ---------------------------------------------------------------------------
# Library special case: torch float64 SDPA on the CPU
# ---------------------------------------------------------------------------

def _sdpa(q, k, v, scale, causal):
    """q [B,N,Hq,d], k/v [B,M,Hkv,d] float64 numpy -> O [B,N,Hq,d]."""
    qt = torch.from_numpy(np.ascontiguousarray(q)).permute(0, 2, 1, 3)
    kt = torch.from_numpy(np.ascontiguousarray(k)).permute(0, 2, 1, 3)
    vt = torch.from_numpy(np.ascontiguousarray(v)).permute(0, 2, 1, 3)
    g = qt.shape[1] // kt.shape[1]
    kt = kt.repeat_interleave(g, dim=1)
    vt = vt.repeat_interleave(g, dim=1)
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=causal,
                                                         scale=scale)
    return o.permute(0, 2, 1, 3).numpy()


def check_sdpa(ora):
    for i, (B, N, Hq, Hkv, d, causal) in enumerate([(2, 33, 4, 2, 16, True), (1, 40, 6, 3, 8, False),
                                                    (1, 64, 8, 1, 32, True)]):
        q = _rand((B, N, Hq, d), 70 + i)
        k = _rand((B, N, Hkv, d), 80 + i)
        v = _rand((B, N, Hkv, d), 90 + i)
        O, _ = ora.attn_ref(q, k, v, 0.25, causal)
        _close(O, _sdpa(q, k, v, 0.25, causal), 1e-12, f"sdpa case {i}")
    # causal with N < M: SDPA with an explicit boolean mask (key j allowed for
    # query i when j <= i + M - N), since its is_causal flag is top-left only
    B, N, M, Hq, Hkv, d = 2, 7, 19, 4, 2, 8
    q, k, v = _rand((B, N, Hq, d), 75), _rand((B, M, Hkv, d), 85), _rand((B, M, Hkv, d), 95)
    O, _ = ora.attn_ref(q, k, v, 0.3, True)
    qt = torch.from_numpy(q).permute(0, 2, 1, 3)
    kt = torch.from_numpy(k).permute(0, 2, 1, 3).repeat_interleave(Hq // Hkv, dim=1)
    vt = torch.from_numpy(v).permute(0, 2, 1, 3).repeat_interleave(Hq // Hkv, dim=1)
    allow = torch.arange(M)[None, :] <= torch.arange(N)[:, None] + (M - N)
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=allow, scale=0.3)
    _close(O, o.permute(0, 2, 1, 3).numpy(), 1e-12, "sdpa bottom-right mask")


def check_causal_chunk_is_tail_of_full(ora):
    """Causal attention of the last N query positions against all M keys
    equals the same rows of the full-length (N = M) causal attention, and the
    last query sees every key (its row equals non-causal attention)."""
    B, M, Hq, Hkv, d = 2, 13, 4, 2, 6
    qf, k, v = _rand((B, M, Hq, d), 160), _rand((B, M, Hkv, d), 161), _rand((B, M, Hkv, d), 162)
    Of, Lf = ora.attn_ref(qf, k, v, 0.45, True)
    for N in (1, 4, M):
        O, L = ora.attn_ref(qf[:, M - N:], k, v, 0.45, True)
        _close(O, Of[:, M - N:], what=f"chunk of {N} rows: O")
        _close(L, Lf[:, :, M - N:], what=f"chunk of {N} rows: lse")
    On, Ln = ora.attn_ref(qf[:, M - 1:], k, v, 0.45, False)
    _close(Of[:, M - 1:], On, what="last row sees every key: O")
    _close(Lf[:, :, M - 1:], Ln, what="last row sees every key: lse")


# ---------------------------------------------------------------------------
# Closed forms and invariants
# ---------------------------------------------------------------------------

def check_identity_v_rows_are_probabilities(ora):
    """With V = identity (d = M), O is the probability matrix: entries >= 0,
    rows sum to 1, causal rows vanish above the diagonal, and each row equals
    exp(S_ij - lse_i)."""
    for causal in (False, True):
        B, N, H, d = 1, 12, 2, 5
        q = _rand((B, N, H, d), 100)
        k = _rand((B, N, H, d), 101)
        v = np.broadcast_to(np.eye(N)[None, :, None, :], (B, N, H, N)).copy()
        P, lse = ora.attn_ref(q, k, v, 0.8, causal)
        assert np.all(P >= 0)
        _close(P.sum(-1), np.ones((B, N, H)), what="row sums")
        if causal:
            iu = np.triu_indices(N, 1)
            assert np.all(P[0][iu[0], :, iu[1]] == 0), "causal probabilities above diagonal"
        S = 0.8 * np.einsum("bihd,bjhd->bhij", q, k)
        expected = np.exp(S - lse[..., None])
        if causal:
            expected = np.where(np.triu(np.ones((N, N), bool), 1), 0.0, expected)
        _close(P.transpose(0, 2, 1, 3), expected, what="P = exp(S - lse)")


def check_constant_v(ora):
    B, N, Hq, Hkv, d = 2, 9, 4, 2, 6
    q, k = _rand((B, N, Hq, d), 110), _rand((B, N, Hkv, d), 111)
    u = _rand((d,), 112)
    v = np.broadcast_to(u, (B, N, Hkv, d)).copy()
    for causal in (False, True):
        O, _ = ora.attn_ref(q, k, v, 0.5, causal)
        _close(O, np.broadcast_to(u, O.shape), what="constant V")


def check_single_key(ora):
    B, Hq, d = 2, 3, 7
    q, k, v = _rand((B, 1, Hq, d), 120), _rand((B, 1, Hq, d), 121), _rand((B, 1, Hq, d), 122)
    for causal in (False, True):
        O, lse = ora.attn_ref(q, k, v, 0.4, causal)
        _close(O, v, what="M=1 output")
        _close(lse[:, :, 0], 0.4 * np.sum(q[:, 0] * k[:, 0], -1), what="M=1 lse")


def check_causal_row0(ora):
    B, N, Hq, Hkv, d = 2, 11, 4, 2, 5
    q, k, v = _rand((B, N, Hq, d), 130), _rand((B, N, Hkv, d), 131), _rand((B, N, Hkv, d), 132)
    O, lse = ora.attn_ref(q, k, v, 0.6, True)
    kv = np.repeat(np.arange(Hkv), Hq // Hkv)
    _close(O[:, 0], v[:, 0][:, kv], what="causal row 0 output")
    _close(lse[:, :, 0], 0.6 * np.sum(q[:, 0] * k[:, 0][:, kv], -1), what="causal row 0 lse")


def check_zero_scale(ora):
    """scale = 0: uniform weights over the allowed keys."""
    B, N, Hq, d = 1, 8, 2, 3
    q, k, v = _rand((B, N, Hq, d), 140), _rand((B, N, Hq, d), 141), _rand((B, N, Hq, d), 142)
    O, lse = ora.attn_ref(q, k, v, 0.0, False)
    _close(O, np.broadcast_to(v.mean(1, keepdims=True), O.shape), what="scale 0 output")
    _close(lse, np.full(lse.shape, math.log(N)), what="scale 0 lse")
    O, lse = ora.attn_ref(q, k, v, 0.0, True)
    cum = np.cumsum(v, axis=1) / np.arange(1, N + 1)[None, :, None, None]
    _close(O, cum, what="causal scale 0 output")
    _close(lse, np.broadcast_to(np.log(np.arange(1, N + 1)), lse.shape), what="causal scale 0 lse")


def check_key_shift(ora):
    """Adding u to every key leaves O unchanged and shifts lse_i by scale*q_i.u."""
    B, N, Hq, d = 1, 10, 2, 4
    q, k, v = _rand((B, N, Hq, d), 150), _rand((B, N, Hq, d), 151), _rand((B, N, Hq, d), 152)
    u = _rand((d,), 153)
    for causal in (False, True):
        O0, l0 = ora.attn_ref(q, k, v, 0.7, causal)
        O1, l1 = ora.attn_ref(q, k + u, v, 0.7, causal)
        _close(O1, O0, what="key shift output")
        _close(l1 - l0, 0.7 * np.einsum("bihd,d->bhi", q, u), what="key shift lse")


def check_permutation(ora):
    B, N, M, Hq, d = 1, 6, 13, 2, 4
    q, k, v = _rand((B, N, Hq, d), 160), _rand((B, M, Hq, d), 161), _rand((B, M, Hq, d), 162)
    perm = np.random.default_rng(163).permutation(M)
    O0, l0 = ora.attn_ref(q, k, v, 0.5, False)
    O1, l1 = ora.attn_ref(q, k[:, perm], v[:, perm], 0.5, False)
    _close(O1, O0, what="permutation output")
    _close(l1, l0, what="permutation lse")


def check_gqa_is_repeated_mha(ora):
    B, N, Hq, Hkv, d = 2, 9, 6, 2, 4
    q, k, v = _rand((B, N, Hq, d), 170), _rand((B, N, Hkv, d), 171), _rand((B, N, Hkv, d), 172)
    g = Hq // Hkv
    for causal in (False, True):
        O0, l0 = ora.attn_ref(q, k, v, 0.5, causal)
        O1, l1 = ora.attn_ref(q, np.repeat(k, g, axis=2), np.repeat(v, g, axis=2), 0.5, causal)
        _close(O0, O1, what="GQA output")
        _close(l0, l1, what="GQA lse")


def check_decode_is_single_query_attention(ora):
    B, Hq, Hkv, M, d = 2, 4, 2, 37, 6
    q, k, v = _rand((B, Hq, d), 180), _rand((B, Hkv, M, d), 181), _rand((B, Hkv, M, d), 182)
    O, L, _, _ = ora.decode_ref(q, k, v, 0.45, 8)
    Of, Lf = ora.attn_ref(q[:, None], k.transpose(0, 2, 1, 3), v.transpose(0, 2, 1, 3), 0.45, False)
    _close(O, Of[:, 0], what="decode vs forward output")
    _close(L, Lf[:, :, 0], what="decode vs forward lse")


def check_merge_identities(ora):
    B, Hq, M, d = 1, 3, 29, 5
    q, k, v = _rand((B, Hq, d), 190), _rand((B, Hq, M, d), 191), _rand((B, Hq, M, d), 192)
    ref = None
    for chunk in (1, 3, 7, 29, 64):          # any partition, uneven tail included
        O, L, op, lp = ora.decode_ref(q, k, v, 0.5, chunk)
        if ref is None:
            ref = (O, L)
        _close(O, ref[0], what=f"partition {chunk} output")
        _close(L, ref[1], what=f"partition {chunk} lse")
        rev = ora.lse_merge_ref(op[..., ::-1, :], lp[..., ::-1])   # order invariance
        _close(rev[0], O, what="reversed chunk order")
    op1, lp1 = ora.decode_partials_ref(q, k, v, 0.5, M)          # one chunk: identity merge
    O1, L1 = ora.lse_merge_ref(op1, lp1)
    _close(O1, op1[..., 0, :], what="single chunk output")
    _close(L1, lp1[..., 0], what="single chunk lse")
    # two chunks with equal lse average their outputs
    o2 = _rand((2, 4), 193)
    Om, Lm = ora.lse_merge_ref(o2[None], np.array([[0.3, 0.3]]))
    _close(Om[0], o2.mean(0), what="equal-weight merge")
    _close(Lm[0], 0.3 + math.log(2.0), what="equal-weight merge lse")
    # a row with no key at all (every chunk empty): the empty sum, O = 0 and
    # lse = -inf; a non-empty row next to it is unaffected
    Oe, Le = ora.lse_merge_ref(np.stack([o2, o2]), np.array([[-np.inf, -np.inf], [0.3, -np.inf]]))
    _close(Oe[0], np.zeros(4), tol=0.0, what="empty-row merge output")
    assert Le[0] == -np.inf, f"empty-row merge lse {Le[0]}"
    _close(Oe[1], o2[0], what="merge with one empty chunk")
    _close(Le[1], 0.3, what="merge with one empty chunk lse")
    # a NaN partial is not an empty row: NaN propagates to O and lse
    with np.errstate(invalid="ignore"):
        On, Ln = ora.lse_merge_ref(o2[None], np.array([[np.nan, -np.inf]]))
    assert np.isnan(Ln[0]) and np.all(np.isnan(On[0])), f"NaN partial merged as {On[0]}, {Ln[0]}"


def check_two_keys_closed_form(ora):
    """Two keys: O = sigmoid-weighted mix, lse = log(e^s0 + e^s1)."""
    q = np.array([[[[1.0, -2.0]]]])
    k = np.array([[[[0.5, 0.25]], [[-1.0, 3.0]]]])
    v = np.array([[[[2.0, 1.0]], [[-4.0, 0.5]]]])
    s0, s1 = 0.9 * (0.5 - 0.5), 0.9 * (-1.0 - 6.0)
    w1 = 1.0 / (1.0 + math.exp(s0 - s1))
    O, lse = ora.attn_ref(q, k, v, 0.9, False)
    _close(O[0, 0, 0], [(1 - w1) * 2.0 + w1 * -4.0, (1 - w1) * 1.0 + w1 * 0.5], what="two-key O")
    _close(lse[0, 0, 0], math.log(math.exp(s0) + math.exp(s1)), what="two-key lse")


def _pages(k, bs, seed):
    """Store contiguous K [B, Hkv, M, d] in pages [num_blocks, bs, Hkv, d] in a
    shuffled page order (plus one unused page); returns (cache, block_table)."""
    B, Hkv, M, d = k.shape
    nblk = -(-M // bs)
    order = np.random.default_rng(seed).permutation(B * nblk + 1)
    cache = _rand((B * nblk + 1, bs, Hkv, d), seed + 1)   # unused rows hold noise
    table = np.zeros((B, nblk), dtype=np.int64)
    for b in range(B):
        for j in range(nblk):
            p = order[b * nblk + j]
            table[b, j] = p
            rows = k[b, :, j * bs:(j + 1) * bs].transpose(1, 0, 2)   # [rows, Hkv, d]
            cache[p, :rows.shape[0]] = rows
    return cache, table


def check_paged_decode_is_decode_of_gathered_keys(ora):
    """Keys stored in shuffled pages decode exactly like the contiguous keys."""
    B, Hq, Hkv, M, d, bs = 2, 4, 2, 37, 5, 8
    q, k, v = _rand((B, Hq, d), 300), _rand((B, Hkv, M, d), 301), _rand((B, Hkv, M, d), 302)
    kc, bt = _pages(k, bs, 303)
    vc, bt2 = _pages(v, bs, 303)
    assert (bt == bt2).all()
    for chunk in (4, 16, 64):
        O, L, op, lp = ora.paged_decode_ref(q, kc, vc, bt, np.full(B, M), 0.6, chunk)
        Or, Lr, opr, lpr = ora.decode_ref(q, k, v, 0.6, chunk)
        _close(O, Or, what=f"paged output, chunk {chunk}")
        _close(L, Lr, what=f"paged lse, chunk {chunk}")
        _close(op[:, :, :opr.shape[2]], opr, what=f"paged partials, chunk {chunk}")


def check_paged_decode_variable_lengths(ora):
    """Sequence b with seq_lens[b] keys decodes like its truncated keys; chunks
    past the end carry no weight."""
    B, Hq, Hkv, M, d, bs = 3, 2, 1, 40, 4, 8
    q, k, v = _rand((B, Hq, d), 310), _rand((B, Hkv, M, d), 311), _rand((B, Hkv, M, d), 312)
    kc, bt = _pages(k, bs, 313)
    vc, _ = _pages(v, bs, 313)
    lens = np.array([1, 17, 40])
    O, L, op, lp = ora.paged_decode_ref(q, kc, vc, bt, lens, 0.7, 16)
    assert op.shape[2] == 3
    # an empty sequence has no key: O = 0, lse = -inf (the empty sum)
    Oz, Lz, opz, lpz = ora.paged_decode_ref(q, kc, vc, bt, np.array([0, 17, 40]), 0.7, 16)
    _close(Oz[0], np.zeros((Hq, d)), tol=0.0, what="empty sequence output")
    assert np.all(Lz[0] == -np.inf) and np.all(lpz[0] == -np.inf), "empty sequence lse"
    _close(Oz[1:], O[1:], what="other sequences next to an empty one")
    for b, n in enumerate(lens):
        Or, Lr, opr, lpr = ora.decode_ref(q[b:b + 1], k[b:b + 1, :, :n], v[b:b + 1, :, :n], 0.7, 16)
        _close(O[b], Or[0], what=f"seq {b} output")
        _close(L[b], Lr[0], what=f"seq {b} lse")
        nc = opr.shape[2]
        assert np.all(lp[b, :, nc:] == -np.inf) and np.all(op[b, :, nc:] == 0.0), "empty chunks"


def check_e4m3_decode(ora):
    """The E4M3 decoder against torch's float8_e4m3fn on all 256 codes, and
    values the format fixes."""
    codes = np.arange(256, dtype=np.uint8)
    mine = ora.e4m3_decode(codes)
    lib = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    assert np.array_equal(np.isnan(mine), np.isnan(lib)), "NaN codes"
    ok = ~np.isnan(lib)
    _close(mine[ok], lib[ok], tol=0.0, what="e4m3 values")
    fixed = {0x00: 0.0, 0x38: 1.0, 0x01: 2.0 ** -9, 0x08: 2.0 ** -6, 0x7E: 448.0, 0xFE: -448.0, 0x41: 2.25}
    for c, val in fixed.items():
        _close(ora.e4m3_decode(np.array([c], dtype=np.uint8)), [val], tol=0.0, what=f"code {c:#x}")


def check_fp8kv_decode_is_decode_of_scaled_values(ora):
    B, Hq, Hkv, M, d = 2, 4, 2, 21, 5
    q = _rand((B, Hq, d), 400)
    g = np.random.default_rng(401)
    kc = g.integers(0, 256, (B, Hkv, M, d)).astype(np.uint8)
    vc = g.integers(0, 256, (B, Hkv, M, d)).astype(np.uint8)
    kc[(kc & 0x7F) == 0x7F] = 0x10     # no NaN codes
    vc[(vc & 0x7F) == 0x7F] = 0x22
    lib = lambda c: torch.from_numpy(c).view(torch.float8_e4m3fn).double().numpy()
    ks, vs = float(np.float32(0.02)), 3.0    # the fp32 scales a caller hands over
    O, L, op, lp = ora.decode_fp8kv_ref(q, kc, vc, ks, vs, 0.5, 8)
    Or, Lr, opr, lpr = ora.decode_ref(q, lib(kc) * ks, lib(vc) * vs, 0.5, 8)
    _close(O, Or, what="fp8 kv output")
    _close(L, Lr, what="fp8 kv lse")
    _close(op, opr, what="fp8 kv partials")


def check_fp8qk_is_attention_of_scaled_values(ora):
    """FP8 Q/K attention equals torch's float64 SDPA on torch's decoding of the
    codes times the scales (causal GQA and non-causal MHA)."""
    lib = lambda c: torch.from_numpy(c).view(torch.float8_e4m3fn).double()
    g = np.random.default_rng(410)
    for B, N, M, Hq, Hkv, d, causal in [(1, 9, 9, 4, 2, 8, True), (2, 5, 11, 2, 2, 6, False)]:
        qc = g.integers(0, 256, (B, N, Hq, d)).astype(np.uint8)
        kc = g.integers(0, 256, (B, M, Hkv, d)).astype(np.uint8)
        qc[(qc & 0x7F) >= 0x60] &= 0x3F     # no NaN codes, moderate magnitudes
        kc[(kc & 0x7F) >= 0x60] &= 0x3F
        v = _rand((B, M, Hkv, d), 411)
        qs, ks = float(np.float32(0.03)), float(np.float32(0.05))
        O, L = ora.attn_fp8qk_ref(qc, kc, v, qs, ks, 0.7, causal)
        qd, kd = (lib(qc) * qs).numpy(), (lib(kc) * ks).numpy()
        _close(O, _sdpa(qd, kd, v, 0.7, causal), what=f"fp8 qk output {causal}")
        # lse: torch's logsumexp of the masked scores of the decoded values
        qt = torch.from_numpy(qd).permute(0, 2, 1, 3)
        kt = torch.from_numpy(kd).permute(0, 2, 1, 3).repeat_interleave(Hq // Hkv, dim=1)
        S = 0.7 * qt @ kt.transpose(-1, -2)
        if causal:
            S = S.masked_fill(torch.arange(M)[None, :] > torch.arange(N)[:, None] + (M - N), float("-inf"))
        _close(L, torch.logsumexp(S, dim=-1).numpy(), what=f"fp8 qk lse {causal}")


FAST_CHECKS = [
    check_brute_prefill_tiny, check_brute_decode_tiny, check_sdpa,
    check_identity_v_rows_are_probabilities, check_constant_v, check_single_key,
    check_causal_row0, check_zero_scale, check_key_shift, check_permutation,
    check_gqa_is_repeated_mha, check_decode_is_single_query_attention,
    check_merge_identities, check_two_keys_closed_form, check_causal_chunk_is_tail_of_full,
    check_paged_decode_is_decode_of_gathered_keys, check_paged_decode_variable_lengths,
    check_e4m3_decode, check_fp8kv_decode_is_decode_of_scaled_values, check_fp8qk_is_attention_of_scaled_values,
]


def failing_checks(ora):
    """Names of the fast checks that the given oracle fails (exceptions count)."""
    bad = []
    for chk in FAST_CHECKS:
        try:
            chk(ora)
        except Exception as e:  # noqa: BLE001 - a crash is a failed pin too
            bad.append(f"{chk.__name__}: {type(e).__name__}: {e}"[:200])
    return bad
