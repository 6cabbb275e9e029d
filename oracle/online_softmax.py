"""Tiled online-softmax model with a lazy rescaling threshold (fp64 or fp32).

TEST INFRASTRUCTURE (only tests/, ``__graft_entry__.smoke()`` and bench.py's
``cpu_baseline`` leg may use oracle/).  This is the oracle's own model of the
method's streaming step, used to pin the claim that skipping rescales leaves the
result exact; the GPU parity tests compare against ``oracle.attention`` instead.

Streaming softmax (fdeinterviews.com FA4 summary, opening paragraph: queries and
keys are tiled and softmax is computed on the fly while everything stays on
chip): key tiles are visited one at a time; each query row keeps a reference
maximum m, a running sum l and an unnormalised output accumulator acc.

Lazy rescaling (same page, "Lazy rescaling" bullet; lecompute.fr FA4 article,
section "Move some exponential work to different units", last paragraph): the
row's reference maximum is moved -- and l and acc multiplied by the matching
factor -- only when the tile's maximum exceeds the reference by more than
``tau`` in log2 units (tau = 8, a factor of 256).  Otherwise the stale reference
is kept, so the weights of that tile may reach at most 2**tau, which keeps the
running sums finite.  The final division by l fixes the result up; in exact
arithmetic it equals the eager (tau = 0) result.

All exponentials are taken in base 2 on the log2-scaled scores
x = s * scale * log2(e), as the method does.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

LOG2E = 1.0 / math.log(2.0)


@dataclass
class TiledStats:
    rescales: int          # number of (row, tile) steps where the reference moved
    steps: int             # number of (row, tile) steps with at least one visible key
    max_weight: float      # largest un-normalised weight 2**(x - m) seen


def tiled_head_forward(q, k, v, scale: float, causal: bool, block_k: int, tau: float,
                       dtype=np.float64, reverse_tiles: bool = False):
    """One head, streaming over key tiles of ``block_k`` keys with threshold ``tau``.

    Returns (O [Lq,D], LSE [Lq] natural log, TiledStats).  ``dtype`` selects the
    arithmetic precision of the model (float64, or float32 to emulate a kernel's
    accumulators).  ``reverse_tiles`` visits key tiles from last to first.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    lq, lk = q.shape[0], k.shape[0]
    c = dtype(float(scale) * LOG2E)
    m = np.full(lq, -np.inf, dtype=dtype)
    l = np.zeros(lq, dtype=dtype)
    acc = np.zeros((lq, v.shape[1]), dtype=dtype)
    rows = np.arange(lq)
    stats = TiledStats(0, 0, 0.0)
    starts = list(range(0, lk, block_k))
    if reverse_tiles:
        starts = starts[::-1]
    for k0 in starts:
        kk = np.arange(k0, min(lk, k0 + block_k))
        s = (q @ k[kk].T).astype(dtype)
        visible = np.ones_like(s, dtype=bool) if not causal else (kk[None, :] <= rows[:, None] + (lk - lq))
        s = np.where(visible, s, dtype(-np.inf))
        tile_max = s.max(axis=1)                       # -inf when nothing is visible
        has = np.isfinite(tile_max)
        stats.steps += int(has.sum())
        m_new = np.maximum(m, tile_max)
        # log2-unit growth of the reference; a row seeing its first key always moves.
        with np.errstate(invalid="ignore"):
            grow = np.where(np.isfinite(m), (m_new - m) * c, np.inf)
        move = has & (grow > tau)
        stats.rescales += int(move.sum())
        with np.errstate(invalid="ignore"):
            shift = np.where(np.isfinite(m), (m - m_new) * c, -np.inf)
        alpha = np.where(move & np.isfinite(m), np.exp2(shift), dtype(0.0)).astype(dtype)
        alpha = np.where(move, alpha, dtype(1.0)).astype(dtype)
        m = np.where(move, m_new, m)
        l = l * alpha
        acc = acc * alpha[:, None]
        ref = np.where(np.isfinite(m), m, dtype(0.0)) * c
        x = s * c - ref[:, None]
        p = np.where(visible, np.exp2(x), dtype(0.0)).astype(dtype)
        if p.size:
            stats.max_weight = max(stats.max_weight, float(p.max()))
        l = l + p.sum(axis=1, dtype=dtype)
        acc = acc + (p @ v[kk].astype(dtype)).astype(dtype)
    seen = l > 0
    o = np.where(seen[:, None], acc / np.where(seen, l, 1)[:, None], 0.0)
    lse = np.where(seen, (np.where(np.isfinite(m), m, 0) * c + np.log2(np.where(seen, l, 1)))
                   / LOG2E, -np.inf)
    return o.astype(np.float64), lse.astype(np.float64), stats
