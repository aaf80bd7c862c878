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
    tail tiles, and the wave's last tile), which tests it after masking; in
    a max-free pass (below) only on a wave's first tile.

A workgroup (four waves sharing the K/V tiles) first runs a pass whose steps
never move the reference (it stays at the first tile's row max; a general
step sets it only when it is the wave's first).  The weights of tiles that
outgrow the reference are then up to 2^(excess), which P and fp32 hold up to
P's largest value; the pass is rerun with the exact steps when, at its end,
some lane's row sum is 2^100 (bf16 P) or 2^15 (fp16 P) or more, or a weight or
an accumulator overflowed (bf16: fp32's range; fp16: a weight of 65520 or
more, which rounds to Inf in P and leaves an accumulator that is not finite).
The emulation follows each row's sum (over both lanes that share the row) and
its largest weight through the pass, rescales included.

This module replays that control flow on the host in float64 (which rows a
wave owns, which tiles it visits and along which path, the masks, the
ballots and the restart decision) so that a test can show that its inputs
reach each branch before it compares the GPU output with the oracle.  It is
test code: it computes no attention output.
"""
from __future__ import annotations

import math

import numpy as np

BN = 64          # keys per tile
WAVE_ROWS = 32   # query rows per wave
WAVES = 4        # waves per workgroup
BM = 128         # query rows per workgroup
LAZY = 8.0       # log2 units the tile max must exceed the reference by
RESTART = {"bf16": 100.0, "f16": 15.0}  # log2 of a lane's row sum at which the max-free pass is rerun
OVERFLOW = 127.0  # bf16 P: log2 of a weight, row sum or accumulator that may overflow fp32 (|v| < 2)
F16_INF = math.log2(65520.0)  # fp16 P: log2 of the smallest weight that rounds to Inf


def _f64(x):
    return x.detach().double().cpu().numpy() if hasattr(x, "detach") else np.asarray(x, np.float64)


def rescale_events(q, k, scale: float, causal: bool, max_free: bool = False, p_dtype: str = "bf16",
                   margin: float = 0.05):
    """Count the kernel's rescale decisions on inputs q [B,N,Hq,d], k [B,M,Hkv,d].

    ``max_free``: the kernel's first pass runs without a moving reference
    (every head dim; False replays the exact steps alone); ``p_dtype`` ("bf16" or "f16") is
    the type of P, which sets when that pass is rerun.

    Returns a dict of counts of decisions the kernel surely takes (each more
    than ``margin`` log2 units, far beyond the fp32 rounding of the scores,
    away from its threshold):
      ``fast``     (wave, tile) pairs rescaled on the exact steady-state path
                   (the only pass, or the rerun after a restart);
      ``general``  (wave, tile) pairs rescaled on the general path, in the
                   pass whose result is kept;
      ``free_growth`` waves of workgroups that surely keep their max-free
                   pass although a steady tile exceeded the row's reference by
                   more than 8 (where an exact step would have rescaled);
      ``restart``  workgroups that surely rerun with the exact steps;
      ``uncertain`` workgroups too close to the restart threshold to say;
    ``max_jump``, the largest excess of a tile max over its row's reference
    where the step did not rescale (in the pass whose result is kept, or the
    first pass), and
    ``max_lag``, the largest move of a row's reference in a rescale of a kept
    pass (its factor 2^-lag is below fp32's normal range past 126).
    """
    q, k = _f64(q), _f64(k)
    B, N, Hq, d = q.shape
    M, Hkv = k.shape[1], k.shape[2]
    group = Hq // Hkv
    pack = 1
    while pack * 2 * 64 <= BM and group % (pack * 2) == 0:
        pack *= 2
    rows = BM // pack                       # query rows per head in one workgroup
    waves_per_head = WAVES // pack
    c = float(np.float32(float(np.float32(scale)) * math.log2(math.e)))
    off = M - N if causal else 0
    n_qt = -(-N // rows)
    ev = {"fast": 0, "general": 0, "free_growth": 0, "restart": 0, "uncertain": 0, "max_jump": -math.inf,
          "max_lag": -math.inf}
    keys = np.arange(M)

    def run_wave(b, h, qw, q_start, exact):
        """One wave's pass: its fast and general rescale events, the largest
        excess of a tile over the reference where no rescale followed, the
        log2 of the rows' sums at the end and their largest log2 during the
        pass (float64, whose range covers fp32's many times over)."""
        kh = h // group
        Kb = k[b, :, kh, :]
        qi = np.arange(qw, qw + WAVE_ROWS)
        # rows past N load row N-1 (their results are never stored)
        Qw = q[b, np.minimum(qi, N - 1), h, :]
        S = Qw @ Kb.T                       # raw scores [32, M]
        kv_end = min(M, q_start + rows + off) if causal else M
        n_tiles = -(-kv_end // BN)
        qlast = qw + WAVE_ROWS - 1
        wave_tiles = min(n_tiles, (qlast + off) // BN + 1) if causal else n_tiles
        fast_end = min(min(wave_tiles - 1, M // BN), (qw + off + 1) // BN if causal else wave_tiles)
        m_run = np.full(WAVE_ROWS, -math.inf)
        l_row = np.zeros(WAVE_ROWS)
        out = {"fast": 0, "general": 0, "excess": -math.inf, "l_max": -math.inf, "lag": -math.inf,
               "w_max": -math.inf}

        def tile_scores(j, masked):
            t = S[:, j * BN:min((j + 1) * BN, M)] * c
            if masked:
                kk = keys[j * BN:min((j + 1) * BN, M)]
                ok = np.ones_like(t, dtype=bool)
                if causal:
                    ok &= kk[None, :] <= qi[:, None] + off
                t = np.where(ok, t, -math.inf)
            return t

        def ballot(m_tile, path):
            nonlocal m_run, l_row
            finite = np.isfinite(m_run)
            if finite.any():
                jump = np.max((m_tile - m_run)[finite])
                if path == "fast":
                    out["excess"] = max(out["excess"], jump)
                if jump > LAZY + margin:
                    out[path] += 1
            if np.any(m_tile > m_run + LAZY):
                m_new = np.maximum(m_run, m_tile)
                moved = np.isfinite(m_run) & (m_new > m_run)
                if moved.any():
                    out["lag"] = max(out["lag"], float(np.max((m_new - m_run)[moved])))
                alpha = np.where(m_new == -math.inf, 1.0, np.exp2(m_run - np.where(m_new == -math.inf, 0.0, m_new)))
                l_row = l_row * alpha
                m_run = m_new

        def accumulate(t):
            nonlocal l_row
            m_use = np.where(m_run == -math.inf, 0.0, m_run)
            out["w_max"] = max(out["w_max"], float(np.max(t - m_use[:, None])))
            with np.errstate(over="ignore"):  # inf past float64's range: an overflow either way
                l_row = l_row + np.exp2(t - m_use[:, None]).sum(axis=1)
            out["l_max"] = max(out["l_max"], float(np.log2(np.max(l_row))) if np.max(l_row) > 0 else -math.inf)

        for j in range(n_tiles):
            if j < fast_end:
                t = tile_scores(j, False)
                m_tile = t.max(axis=1)
                if j == 0:
                    m_run = m_tile          # the first steady step sets the reference
                elif exact:
                    ballot(m_tile, "fast")
                else:
                    out["excess"] = max(out["excess"], np.max(m_tile - m_run))
                accumulate(t)
            elif j < wave_tiles:
                n0 = j * BN
                need_mask = (causal and n0 + BN - 1 > qw + off) or (n0 + BN > M)
                t = tile_scores(j, need_mask)
                mx = t.max(axis=1)
                if exact or j == 0:
                    ballot(np.where(np.isfinite(mx), mx, -math.inf), "general")
                else:
                    # a max-free pass keeps its reference here too (masked keys weigh 0)
                    ok = np.isfinite(mx) & np.isfinite(m_run)
                    if ok.any():
                        out["excess"] = max(out["excess"], float(np.max((mx - m_run)[ok])))
                accumulate(t)
        out["l_end"] = float(np.log2(np.max(l_row)))
        return out

    for b in range(B):
        for kh in range(Hkv):
            for hp in range(group // pack):
                for qt in range(n_qt):
                    q_start = qt * rows
                    waves = [(kh * group + hp * pack + w // waves_per_head,
                              q_start + (w % waves_per_head) * WAVE_ROWS) for w in range(WAVES)]
                    first = [run_wave(b, h, qw, q_start, exact=not max_free) for h, qw in waves]
                    kept = first
                    if max_free:
                        l_end = max(r["l_end"] for r in first)
                        l_max = max(r["l_max"] for r in first)
                        w_max = max(r["w_max"] for r in first)
                        rs = RESTART[p_dtype]
                        # one of a row's two lanes holds at least half its sum
                        if p_dtype == "bf16":
                            surely = l_end - 1.0 > rs + margin or l_max - 1.0 > OVERFLOW + 2.0
                            never = l_end < rs - margin and l_max < OVERFLOW - 1.0
                        else:
                            surely = l_end - 1.0 > rs + margin or w_max > F16_INF + margin
                            never = l_end < rs - margin and w_max < F16_INF - margin
                        if surely:
                            ev["restart"] += 1
                            kept = [run_wave(b, h, qw, q_start, exact=True) for h, qw in waves]
                        elif never:
                            ev["free_growth"] += sum(r["excess"] > LAZY + margin for r in first)
                        else:
                            ev["uncertain"] += 1
                            kept = None
                    if kept is not None:
                        ev["fast"] += sum(r["fast"] for r in kept)
                        ev["general"] += sum(r["general"] for r in kept)
                        ev["max_jump"] = max(ev["max_jump"], max(r["excess"] for r in kept))
                        ev["max_lag"] = max(ev["max_lag"], max(r["lag"] for r in kept))
                    else:
                        ev["max_jump"] = max(ev["max_jump"], max(r["excess"] for r in first))
    return ev
