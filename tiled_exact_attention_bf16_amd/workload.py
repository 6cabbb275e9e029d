"""Algorithmic work and bytes of one attention call (the measurement convention).

FLOP convention fixed by the FA4 roofline (fdeinterviews.com FA4 summary, second
paragraph): for a 128x128 tile the forward's two matrix products take 1,024
cycles at 8,192 ops per clock, i.e. 2 GEMMs x 2*128*128*128 operations, and the
backward's take 2,560 cycles, i.e. five such GEMMs.  Per visible (query, key)
pair this is 4*d FLOP forward and 10*d FLOP backward.  Causal attention counts
only the visible pairs (L(L+1)/2 per sequence and head), not the work a kernel
spends on masked parts of diagonal tiles.
"""
from __future__ import annotations

from typing import Sequence

FWD_FLOP_PER_PAIR_PER_D = 4
BWD_FLOP_PER_PAIR_PER_D = 10


def visible_pairs(seqlen_q: int, seqlen_k: int, causal: bool) -> int:
    """Number of (query, key) pairs the mask leaves visible in one sequence and head."""
    if seqlen_q <= 0 or seqlen_k <= 0:
        return 0
    if not causal:
        return seqlen_q * seqlen_k
    # key j visible to query i iff j <= i + seqlen_k - seqlen_q (bottom-right aligned):
    # the last n = min(seqlen_q, seqlen_k) queries see seqlen_k - n + 1 ... seqlen_k keys,
    # the earlier queries (only when seqlen_q > seqlen_k) see none
    n = min(seqlen_q, seqlen_k)
    return n * (seqlen_k - n) + n * (n + 1) // 2


def total_pairs(seqlens_q: Sequence[int], seqlens_k: Sequence[int], heads: int, causal: bool) -> int:
    return heads * sum(visible_pairs(int(a), int(b), causal) for a, b in zip(seqlens_q, seqlens_k))


def fwd_flops(seqlens_q, seqlens_k, heads: int, head_dim: int, causal: bool) -> int:
    return FWD_FLOP_PER_PAIR_PER_D * head_dim * total_pairs(seqlens_q, seqlens_k, heads, causal)


def bwd_flops(seqlens_q, seqlens_k, heads: int, head_dim: int, causal: bool) -> int:
    return BWD_FLOP_PER_PAIR_PER_D * head_dim * total_pairs(seqlens_q, seqlens_k, heads, causal)


def fwd_min_bytes(total_q: int, total_k: int, heads: int, head_dim: int) -> int:
    """Compulsory HBM bytes of the forward: read Q, K, V (bf16), write O (bf16) and LSE (fp32)."""
    return heads * (total_q * head_dim * 2 * 2 + total_k * head_dim * 2 * 2 + total_q * 4)


def bwd_min_bytes(total_q: int, total_k: int, heads: int, head_dim: int, grad_bytes: int = 4) -> int:
    """Compulsory HBM bytes of the backward: read Q,K,V,O,dO (bf16), LSE (fp32);
    write dQ, dK, dV (``grad_bytes`` each)."""
    reads = heads * (total_q * head_dim * 2 * 3 + total_k * head_dim * 2 * 2 + total_q * 4)
    writes = heads * (total_q + 2 * total_k) * head_dim * grad_bytes
    return reads + writes
