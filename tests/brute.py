"""Pure-Python brute-force attention (independent of the oracle and of numpy).

Each output element is computed from its textbook definition with scalar
Python floats, ``math.exp`` and ``math.fsum`` (exactly rounded sums), so it
shares neither code nor summation order with the numpy oracle.  Used to pin
the oracle on tiny inputs and on the whole of the two small workloads.
"""
from __future__ import annotations

import math


def _tolist(x):
    if hasattr(x, "detach"):
        x = x.detach().double().tolist()
    elif hasattr(x, "tolist"):
        x = x.tolist()
    return x


def brute_attention(q, k, v, scale, causal):
    """q [B][N][Hq][d], k/v [B][M][Hkv][d] nested lists (or arrays/tensors).
    Returns (O [B][N][Hq][d], lse [B][Hq][N]) as nested lists of floats."""
    q, k, v = _tolist(q), _tolist(k), _tolist(v)
    B, N, Hq, d = len(q), len(q[0]), len(q[0][0]), len(q[0][0][0])
    M, Hkv = len(k[0]), len(k[0][0])
    g = Hq // Hkv
    O = [[[[0.0] * d for _ in range(Hq)] for _ in range(N)] for _ in range(B)]
    L = [[[0.0] * N for _ in range(Hq)] for _ in range(B)]
    for b in range(B):
        for h in range(Hq):
            kh = h // g
            for i in range(N):
                # causal: query i is position i + M - N of the key sequence
                allowed = [j for j in range(M) if (not causal) or j <= i + M - N]
                s = {j: scale * math.fsum(q[b][i][h][t] * k[b][j][kh][t] for t in range(d))
                     for j in allowed}
                mx = max(s.values())
                e = {j: math.exp(s[j] - mx) for j in allowed}
                den = math.fsum(e.values())
                for t in range(d):
                    O[b][i][h][t] = math.fsum(e[j] * v[b][j][kh][t] for j in allowed) / den
                L[b][h][i] = mx + math.log(den)
    return O, L


def brute_decode_partials(q, k, v, scale, chunk):
    """q [B][Hq][d], k/v [B][Hkv][M][d].  Returns o_part [B][Hq][C][d] and
    lse_part [B][Hq][C], each chunk's normalised output and log-sum-exp."""
    q, k, v = _tolist(q), _tolist(k), _tolist(v)
    B, Hq, d = len(q), len(q[0]), len(q[0][0])
    Hkv, M = len(k[0]), len(k[0][0])
    g = Hq // Hkv
    C = (M + chunk - 1) // chunk
    op = [[[[0.0] * d for _ in range(C)] for _ in range(Hq)] for _ in range(B)]
    lp = [[[0.0] * C for _ in range(Hq)] for _ in range(B)]
    for b in range(B):
        for h in range(Hq):
            kh = h // g
            for c in range(C):
                js = range(c * chunk, min(M, (c + 1) * chunk))
                s = {j: scale * math.fsum(q[b][h][t] * k[b][kh][j][t] for t in range(d)) for j in js}
                mx = max(s.values())
                e = {j: math.exp(s[j] - mx) for j in js}
                den = math.fsum(e.values())
                for t in range(d):
                    op[b][h][c][t] = math.fsum(e[j] * v[b][kh][j][t] for j in js) / den
                lp[b][h][c] = mx + math.log(den)
    return op, lp


def brute_decode(q, k, v, scale):
    """Unsplit single-query attention: O [B][Hq][d], lse [B][Hq]."""
    q, k, v = _tolist(q), _tolist(k), _tolist(v)
    B, Hq, d = len(q), len(q[0]), len(q[0][0])
    Hkv, M = len(k[0]), len(k[0][0])
    g = Hq // Hkv
    O = [[[0.0] * d for _ in range(Hq)] for _ in range(B)]
    L = [[0.0] * Hq for _ in range(B)]
    for b in range(B):
        for h in range(Hq):
            kh = h // g
            s = [scale * math.fsum(q[b][h][t] * k[b][kh][j][t] for t in range(d)) for j in range(M)]
            mx = max(s)
            e = [math.exp(x - mx) for x in s]
            den = math.fsum(e)
            for t in range(d):
                O[b][h][t] = math.fsum(e[j] * v[b][kh][j][t] for j in range(M)) / den
            L[b][h] = mx + math.log(den)
    return O, L
