"""fp64 CPU oracle for exact scaled-dot-product attention, forward and backward.

TEST INFRASTRUCTURE.  Only tests/, ``__graft_entry__.smoke()`` and bench.py's
``cpu_baseline`` leg may import or call anything under oracle/.  The HIP library
and its Python binding never use it, and this module shares no code with them.

What is computed (the plain definition; every step is a library matmul, exp,
max or sum over whole rows, with no tiling, fusion or reordering beyond
splitting the query rows into independent blocks to bound memory):

  Forward (lecompute.fr FA4 article, section "Between the matrix products the
  kernel must produce weights": queries are compared with keys to give scores, a
  softmax turns each row of scores into positive weights summing to one, and a
  second product combines the values with those weights):
      s_ij  = scale * sum_d q_id k_jd
      s_ij  = -inf where the mask hides key j from query i
      P_ij  = exp(s_ij - m_i) / sum_j exp(s_ij - m_i),  m_i = max_j s_ij
      O_i   = sum_j P_ij v_j
      LSE_i = m_i + ln sum_j exp(s_ij - m_i)      (natural log, scale included)

  Masks (fdeinterviews.com FA4 summary, features paragraph: causal masks and
  variable lengths):  causal hides key j from query i when j > i + (Lk - Lq), so
  that the last query sees every key (the diagonal is aligned to the bottom-right
  corner; with Lq = Lk this is the usual j > i, and with Lq < Lk the queries are
  the last Lq positions of the key sequence, as in generation with a cache);
  variable length restricts attention to the keys of the query's own sequence.
  A query that sees no key gets O = 0, LSE = -inf.

  Backward (the gradient of the forward above; the pages name a backward pass
  and its dQ accumulation but print no equations), from the exact P:
      D_i   = sum_d dO_id O_id
      dV_j  = sum_i P_ij dO_i
      dP_ij = dO_i . v_j
      dS_ij = P_ij (dP_ij - D_i)
      dQ_i  = scale * sum_j dS_ij k_j
      dK_j  = scale * sum_i dS_ij q_i

Inputs are float64 arrays (exact widenings of the bf16 inputs); ``scale`` is the
fp32 value handed to the kernel, widened.
"""
from __future__ import annotations

from typing import Optional, Sequence, Tuple

import numpy as np

ROW_BLOCK = 512


def _mask_block(rows: np.ndarray, n_queries: int, n_keys: int, causal: bool) -> np.ndarray:
    """Return a boolean array, True where key j is visible to the query in ``rows``
    (causal: j <= row + n_keys - n_queries)."""
    if not causal:
        return np.ones((len(rows), n_keys), dtype=bool)
    keys = np.arange(n_keys)
    return keys[None, :] <= rows[:, None] + (n_keys - n_queries)


def head_forward(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float, causal: bool,
                 rows: Optional[Sequence[int]] = None) -> Tuple[np.ndarray, np.ndarray]:
    """Attention for one sequence and one head.

    q: [Lq, D], k and v: [Lk, D] (float64).  ``rows`` optionally selects query
    rows (by index into q) to evaluate; default all.  Returns (O [n, D], LSE [n]).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    lq, d = q.shape
    lk = k.shape[0]
    row_idx = np.arange(lq) if rows is None else np.asarray(rows, dtype=np.int64)
    o = np.zeros((len(row_idx), v.shape[1]), dtype=np.float64)
    lse = np.full(len(row_idx), -np.inf, dtype=np.float64)
    if lk == 0 or len(row_idx) == 0:
        return o, lse
    scale = float(scale)
    for b0 in range(0, len(row_idx), ROW_BLOCK):
        r = row_idx[b0:b0 + ROW_BLOCK]
        s = scale * (q[r] @ k.T)
        vis = _mask_block(r, lq, lk, causal)
        s = np.where(vis, s, -np.inf)
        m = s.max(axis=1)
        seen = np.isfinite(m)
        m_safe = np.where(seen, m, 0.0)
        e = np.exp(s - m_safe[:, None])          # exp(-inf) = 0 for hidden keys
        l = e.sum(axis=1)
        l_safe = np.where(seen, l, 1.0)
        o[b0:b0 + len(r)] = np.where(seen[:, None], (e @ v) / l_safe[:, None], 0.0)
        lse[b0:b0 + len(r)] = np.where(seen, m_safe + np.log(l_safe), -np.inf)
    return o, lse


def head_probabilities(q: np.ndarray, k: np.ndarray, scale: float, causal: bool) -> np.ndarray:
    """The full softmax matrix P [Lq, Lk] for one head (small shapes only)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    rows = np.arange(q.shape[0])
    s = float(scale) * (q @ k.T)
    s = np.where(_mask_block(rows, q.shape[0], k.shape[0], causal), s, -np.inf)
    m = s.max(axis=1)
    seen = np.isfinite(m)
    e = np.exp(s - np.where(seen, m, 0.0)[:, None])
    l = e.sum(axis=1)
    return np.where(seen[:, None], e / np.where(seen, l, 1.0)[:, None], 0.0)


def head_backward(q: np.ndarray, k: np.ndarray, v: np.ndarray, do: np.ndarray, scale: float,
                  causal: bool, o: Optional[np.ndarray] = None) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Gradients (dQ, dK, dV) of one head's attention for the output gradient dO.

    O and LSE are recomputed here in fp64 from the inputs (never taken from a
    GPU run), then P is rebuilt block by block from LSE.  ``o``, when given, is
    the forward output as the backward receives it (e.g. rounded to bf16) and
    enters only D_i = sum_d dO_id O_id, as it does in a backward that reads the
    saved output; by default D uses the exact O.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    lq, lk = q.shape[0], k.shape[0]
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    if lq == 0 or lk == 0:
        return dq, dk, dv
    o_exact, lse = head_forward(q, k, v, scale, causal)
    dvec = (do * (o_exact if o is None else np.asarray(o, dtype=np.float64))).sum(axis=1)
    scale = float(scale)
    for b0 in range(0, lq, ROW_BLOCK):
        r = np.arange(b0, min(lq, b0 + ROW_BLOCK))
        s = scale * (q[r] @ k.T)
        vis = _mask_block(r, lq, lk, causal)
        seen = np.isfinite(lse[r])
        p = np.where(vis & seen[:, None], np.exp(s - np.where(seen, lse[r], 0.0)[:, None]), 0.0)
        dv += p.T @ do[r]
        dp = do[r] @ v.T
        ds = p * (dp - dvec[r][:, None])
        dq[r] = scale * (ds @ k)
        dk += scale * (ds.T @ q[r])
    return dq, dk, dv


# ---- whole-tensor wrappers over the [B,S,H,D] and packed [T,H,D] layouts ----

def _sequences(q_shape, cu_seqlens):
    if cu_seqlens is None:
        return [(b, None, None) for b in range(q_shape[0])]
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    return [(b, int(cu[b]), int(cu[b + 1])) for b in range(len(cu) - 1)]


def forward(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float, causal: bool,
            cu_seqlens: Optional[np.ndarray] = None,
            heads: Optional[Sequence[int]] = None) -> Tuple[np.ndarray, np.ndarray]:
    """Forward over a whole batch.

    Fixed length: q [B,Sq,H,D], k/v [B,Sk,H,D] -> O [B,Sq,H,D], LSE [B,H,Sq].
    Packed variable length (cu_seqlens given, same lengths for Q and K):
    q/k/v [T,H,D] -> O [T,H,D], LSE [H,T].
    ``heads`` restricts the work to some heads (others stay O=0, LSE=-inf).
    """
    h_all = q.shape[-2]
    hs = range(h_all) if heads is None else heads
    o = np.zeros(q.shape[:-1] + (v.shape[-1],), dtype=np.float64)
    if cu_seqlens is None:
        lse = np.full((q.shape[0], h_all, q.shape[1]), -np.inf)
        for b in range(q.shape[0]):
            for h in hs:
                o[b, :, h], lse[b, h] = head_forward(q[b, :, h], k[b, :, h], v[b, :, h], scale, causal)
    else:
        lse = np.full((h_all, q.shape[0]), -np.inf)
        for _, s0, s1 in _sequences(q.shape, cu_seqlens):
            for h in hs:
                o[s0:s1, h], lse[h, s0:s1] = head_forward(q[s0:s1, h], k[s0:s1, h], v[s0:s1, h],
                                                          scale, causal)
    return o, lse


def backward(q: np.ndarray, k: np.ndarray, v: np.ndarray, do: np.ndarray, scale: float,
             causal: bool, cu_seqlens: Optional[np.ndarray] = None,
             heads: Optional[Sequence[int]] = None):
    """Backward over a whole batch; layouts as in ``forward``.  Returns dQ, dK, dV."""
    h_all = q.shape[-2]
    hs = range(h_all) if heads is None else heads
    dq = np.zeros_like(q, dtype=np.float64)
    dk = np.zeros_like(k, dtype=np.float64)
    dv = np.zeros_like(v, dtype=np.float64)
    if cu_seqlens is None:
        for b in range(q.shape[0]):
            for h in hs:
                dq[b, :, h], dk[b, :, h], dv[b, :, h] = head_backward(
                    q[b, :, h], k[b, :, h], v[b, :, h], do[b, :, h], scale, causal)
    else:
        for _, s0, s1 in _sequences(q.shape, cu_seqlens):
            for h in hs:
                dq[s0:s1, h], dk[s0:s1, h], dv[s0:s1, h] = head_backward(
                    q[s0:s1, h], k[s0:s1, h], v[s0:s1, h], do[s0:s1, h], scale, causal)
    return dq, dk, dv
