"""Host emulation of when the prefill kernel moves its reference maximum.

The kernel's online softmax ("fmha sm120: beyond torch.sdpa", section 2: m_i
and l_i rescaled by alpha = exp2(m_old - m_new)) moves a row's reference max
lazily: a wave of 32 query rows rescales only when, for some row, the maximum
of a 64-key tile (scaled to log2 units) exceeds the row's reference by more
than 8.  The tiles go through one of two code paths:

  * the steady-state step (a tile with no masked key whose successor the wave
    still needs), which tests the condition on the tile's row max computed
    during the previous step;
  * the general step (a masked or only first tile, the causal diagonal and
    tail tiles, and the wave's last tile), which tests it after masking.

This module replays that control flow on the host in float64 (which rows a
wave owns, which tiles it visits and along which path, the masks, and the
ballot) so that a test can show that its inputs make both paths rescale
before it compares the GPU output with the oracle.  It is test code: it
computes no attention output.
"""
from __future__ import annotations

import math

import numpy as np

BN = 64          # keys per tile
WAVE_ROWS = 32   # query rows per wave
BM = 128         # query rows per workgroup
LAZY = 8.0       # log2 units the tile max must exceed the reference by


def _f64(x):
    return x.detach().double().cpu().numpy() if hasattr(x, "detach") else np.asarray(x, np.float64)


def rescale_events(q, k, scale: float, causal: bool, margin: float = 0.05):
    """Count the waves' rescale decisions on inputs q [B,N,Hq,d], k [B,M,Hkv,d].

    Returns a dict with the number of (wave, tile) pairs where the kernel
    surely rescales a finite reference (the excess over the reference plus 8
    is above ``margin``, far beyond the fp32 rounding of the scores):
    ``fast`` on the steady-state path, ``general`` on the general path, and
    ``max_jump``, the largest excess of a tile max over its row's reference.
    """
    q, k = _f64(q), _f64(k)
    B, N, Hq, d = q.shape
    M, Hkv = k.shape[1], k.shape[2]
    group = Hq // Hkv
    pack = 1
    while pack * 2 * 64 <= BM and group % (pack * 2) == 0:
        pack *= 2
    rows = BM // pack                       # query rows per head in one workgroup
    c = float(np.float32(float(np.float32(scale)) * math.log2(math.e)))
    off = M - N if causal else 0
    n_qt = -(-N // rows)
    ev = {"fast": 0, "general": 0, "max_jump": -math.inf}
    keys = np.arange(M)
    for b in range(B):
        for h in range(Hq):
            kh = h // group
            Kb = k[b, :, kh, :]
            for qt in range(n_qt):
                q_start = qt * rows
                kv_end = min(M, q_start + rows + off) if causal else M
                n_tiles = -(-kv_end // BN)
                for qw in range(q_start, q_start + rows, WAVE_ROWS):
                    qi = np.arange(qw, qw + WAVE_ROWS)
                    # rows past N load row N-1 (their results are never stored)
                    Qw = q[b, np.minimum(qi, N - 1), h, :]
                    S = Qw @ Kb.T                 # raw scores [32, M]
                    qlast = qw + WAVE_ROWS - 1
                    wave_tiles = min(n_tiles, (qlast + off) // BN + 1) if causal else n_tiles
                    fast_end = min(min(wave_tiles - 1, M // BN), (qw + off + 1) // BN if causal else wave_tiles)
                    m_run = np.full(WAVE_ROWS, -math.inf)

                    def tile_max(j, masked):
                        t = S[:, j * BN:min((j + 1) * BN, M)].copy()
                        if masked:
                            kk = keys[j * BN:min((j + 1) * BN, M)]
                            ok = np.ones_like(t, dtype=bool)
                            if causal:
                                ok &= kk[None, :] <= qi[:, None] + off
                            t = np.where(ok, t, -math.inf)
                        mx = t.max(axis=1)
                        return np.where(np.isfinite(mx), mx * c, -math.inf)

                    def ballot(m_tile, path):
                        nonlocal m_run
                        finite = np.isfinite(m_run)
                        if finite.any():
                            jump = np.max((m_tile - m_run)[finite])
                            ev["max_jump"] = max(ev["max_jump"], jump)
                            if jump > LAZY + margin:
                                ev[path] += 1
                        if np.any(m_tile > m_run + LAZY):
                            m_run = np.maximum(m_run, m_tile)

                    for j in range(n_tiles):
                        if j < fast_end:
                            m_tile = tile_max(j, False)
                            if j == 0:
                                m_run = m_tile    # the first steady step sets the reference
                            else:
                                ballot(m_tile, "fast")
                        elif j < wave_tiles:
                            n0 = j * BN
                            need_mask = (causal and n0 + BN - 1 > qw + off) or (n0 + BN > M)
                            ballot(tile_max(j, need_mask), "general")
    return ev
