"""Seeded synthetic inputs for exact tiled attention.

This module is the one piece shared by the GPU path's tests/bench and the fp64
oracle.  It holds no attention arithmetic: only seeded random draws, the
round-to-nearest-even narrowing of those draws to bfloat16 bit patterns, the
exact widening of the same bit patterns, and the recipe for variable sequence
lengths.  Both sides therefore see identical bf16 inputs.

Workloads follow the regime the pages single out (FlashAttention-4 summary,
fdeinterviews.com, paragraph on long sequences: sequences of several thousand
tokens, often under a causal mask; features paragraph: causal masks and packed
batches of different lengths).  The pages name no public dataset, so every tensor
is drawn i.i.d. from a normal distribution.

Recipe (same for every config):
  rng = numpy.random.default_rng(seed)
  [varlen only] 32 lengths are drawn first (see ``varlen_lengths``)
  then Q, K, V (and dO for backward configs) in that order, each as
  rng.standard_normal(shape, dtype=float32) * std, in logical [B,S,H,D]
  (or packed [T,H,D]) order, narrowed to bf16 by round-to-nearest-even.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

__all__ = [
    "AttnInputs",
    "CONFIGS",
    "f32_to_bf16_bits",
    "bf16_bits_to_f32",
    "bf16_bits_to_f64",
    "varlen_lengths",
    "make_inputs",
    "random_inputs",
    "random_varlen_inputs",
    "random_varlen_qk_inputs",
]


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Narrow float32 values to bf16 bit patterns (uint16), round-to-nearest-even.

    NaN inputs are not expected (draws are finite); they would be kept as NaN.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    out = rounded.astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = 0x7FC0
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def bf16_bits_to_f64(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float64."""
    return bf16_bits_to_f32(b).astype(np.float64)


def _draw_bf16(rng: np.random.Generator, shape, std: float) -> np.ndarray:
    x = rng.standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return f32_to_bf16_bits(x)


def varlen_lengths(rng: np.random.Generator, n: int = 32, total: int = 131072,
                   lo: int = 128, hi: int = 16384) -> np.ndarray:
    """Sequence lengths drawn log-uniform in [lo, hi], then made to sum to ``total``.

    Raw log-uniform draws do not sum to the requested total, so the draws are
    rescaled and clipped to [lo, hi] repeatedly, floored, and the integer residual
    is handed to the longest lengths that still have room below ``hi``.
    """
    if n * lo > total or n * hi < total:
        raise ValueError("total not reachable with n lengths in [lo, hi]")
    u = rng.uniform(math.log(lo), math.log(hi), size=n)
    lens = np.exp(u)
    for _ in range(100):
        lens = np.clip(lens * (total / lens.sum()), lo, hi)
    lens = np.floor(lens).astype(np.int64)
    residual = int(total - lens.sum())
    order = np.argsort(-lens, kind="stable")
    while residual != 0:
        progressed = False
        for i in order:
            if residual > 0 and lens[i] < hi:
                step = min(residual, hi - int(lens[i]))
                lens[i] += step
                residual -= step
                progressed = True
            elif residual < 0 and lens[i] > lo:
                step = min(-residual, int(lens[i]) - lo)
                lens[i] -= step
                residual += step
                progressed = True
            if residual == 0:
                break
        if not progressed:
            raise RuntimeError("could not distribute residual length")
    return lens.astype(np.int32)


@dataclasses.dataclass
class AttnInputs:
    """One attention problem as bf16 bit patterns (uint16 arrays).

    Fixed length: q/k/v/do have shape [B, S, H, D] and cu_seqlens is None.
    Variable length: q/k/v/do have shape [T, H, D] (sequences packed along T) and
    cu_seqlens is the int32 prefix sum of the lengths ([B+1], first entry 0);
    cu_seqlens_k, when given, holds the key/value offsets (else the same as q's).
    """
    name: str
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    scale: float
    causal: bool
    do: Optional[np.ndarray] = None
    cu_seqlens: Optional[np.ndarray] = None
    seed: int = 0
    cu_seqlens_k: Optional[np.ndarray] = None

    @property
    def varlen(self) -> bool:
        return self.cu_seqlens is not None

    @property
    def head_dim(self) -> int:
        return int(self.q.shape[-1])

    @property
    def num_heads(self) -> int:
        return int(self.q.shape[-2])

    @property
    def batch(self) -> int:
        return len(self.cu_seqlens) - 1 if self.varlen else int(self.q.shape[0])

    def seqlens(self) -> np.ndarray:
        if self.varlen:
            return np.diff(self.cu_seqlens).astype(np.int64)
        return np.full(self.q.shape[0], self.q.shape[1], dtype=np.int64)

    def max_seqlen(self) -> int:
        return int(self.seqlens().max()) if self.batch > 0 else 0

    def seqlens_k(self) -> np.ndarray:
        if self.varlen:
            return np.diff(self.cu_seqlens if self.cu_seqlens_k is None else self.cu_seqlens_k).astype(np.int64)
        return np.full(self.k.shape[0], self.k.shape[1], dtype=np.int64)

    def max_seqlen_k(self) -> int:
        return int(self.seqlens_k().max()) if self.batch > 0 else 0

    def sequence(self, b: int, name: str = "q") -> np.ndarray:
        """bf16 bits of one sequence of one tensor, shape [L, H, D]."""
        t = getattr(self, name)
        if self.varlen:
            cu = self.cu_seqlens_k if (name in ("k", "v") and self.cu_seqlens_k is not None) else self.cu_seqlens
            s, e = int(cu[b]), int(cu[b + 1])
            return t[s:e]
        return t[b]


def _fp32_scale(d: int) -> float:
    return float(np.float32(1.0 / math.sqrt(d)))


def random_inputs(seed: int, batch: int, seqlen: int, heads: int, head_dim: int,
                  causal: bool, q_std: float = 1.0, with_do: bool = False,
                  scale: Optional[float] = None, name: str = "random",
                  seqlen_k: Optional[int] = None) -> AttnInputs:
    """Fixed-length problem: Q [B,Sq,H,D], K/V [B,Sk,H,D] (Sk defaults to Sq)."""
    rng = np.random.default_rng(seed)
    sk = seqlen if seqlen_k is None else seqlen_k
    q = _draw_bf16(rng, (batch, seqlen, heads, head_dim), q_std)
    k = _draw_bf16(rng, (batch, sk, heads, head_dim), 1.0)
    v = _draw_bf16(rng, (batch, sk, heads, head_dim), 1.0)
    do = _draw_bf16(rng, (batch, seqlen, heads, head_dim), 1.0) if with_do else None
    sc = _fp32_scale(head_dim) if scale is None else float(np.float32(scale))
    return AttnInputs(name=name, q=q, k=k, v=v, do=do, scale=sc, causal=causal, seed=seed)


def random_varlen_inputs(seed: int, lengths, heads: int, head_dim: int, causal: bool,
                         with_do: bool = False, name: str = "varlen",
                         q_std: float = 1.0) -> AttnInputs:
    """Packed problem with the given per-sequence lengths (Sq = Sk per sequence)."""
    rng = np.random.default_rng(seed)
    lengths = np.asarray(lengths, dtype=np.int64)
    cu = np.zeros(len(lengths) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(lengths)
    t = int(cu[-1])
    q = _draw_bf16(rng, (t, heads, head_dim), q_std)
    k = _draw_bf16(rng, (t, heads, head_dim), 1.0)
    v = _draw_bf16(rng, (t, heads, head_dim), 1.0)
    do = _draw_bf16(rng, (t, heads, head_dim), 1.0) if with_do else None
    return AttnInputs(name=name, q=q, k=k, v=v, do=do, scale=_fp32_scale(head_dim),
                      causal=causal, cu_seqlens=cu, seed=seed)


# The five workloads and the headline forward shape.  Sizes follow the method's
# long-sequence regime; values are synthetic normals.
def random_varlen_qk_inputs(seed: int, q_lengths, k_lengths, heads: int, head_dim: int, causal: bool,
                            name: str = "varlen_qk") -> AttnInputs:
    """Packed problem with separate query and key lengths per sequence."""
    rng = np.random.default_rng(seed)
    q_lengths = np.asarray(q_lengths, dtype=np.int64)
    k_lengths = np.asarray(k_lengths, dtype=np.int64)
    cu_q = np.zeros(len(q_lengths) + 1, dtype=np.int32)
    cu_q[1:] = np.cumsum(q_lengths)
    cu_k = np.zeros(len(k_lengths) + 1, dtype=np.int32)
    cu_k[1:] = np.cumsum(k_lengths)
    q = _draw_bf16(rng, (int(cu_q[-1]), heads, head_dim), 1.0)
    k = _draw_bf16(rng, (int(cu_k[-1]), heads, head_dim), 1.0)
    v = _draw_bf16(rng, (int(cu_k[-1]), heads, head_dim), 1.0)
    return AttnInputs(name=name, q=q, k=k, v=v, scale=_fp32_scale(head_dim), causal=causal, cu_seqlens=cu_q,
                      seed=seed, cu_seqlens_k=cu_k)


CONFIGS = {
    "c1": dict(seed=1, batch=1, seqlen=256, heads=2, head_dim=64, causal=False),
    "c2": dict(seed=2, batch=4, seqlen=4096, heads=16, head_dim=128, causal=False),
    "c2_causal": dict(seed=2, batch=4, seqlen=4096, heads=16, head_dim=128, causal=True),
    "c3": dict(seed=3, batch=1, seqlen=16384, heads=32, head_dim=128, causal=True, q_std=3.0),
    "c4": dict(seed=4, varlen=True, n_seqs=32, total=131072, lo=128, hi=16384,
               heads=16, head_dim=128, causal=True),
    "c5": dict(seed=5, batch=2, seqlen=8192, heads=16, head_dim=128, causal=True, with_do=True),
    "headline": dict(seed=6, batch=2, seqlen=8192, heads=16, head_dim=128, causal=True),
}


def make_inputs(name: str) -> AttnInputs:
    """Build one of the named workloads in ``CONFIGS`` (deterministic in its seed)."""
    cfg = dict(CONFIGS[name])
    seed = cfg.pop("seed")
    if cfg.pop("varlen", False):
        rng = np.random.default_rng(seed)
        lens = varlen_lengths(rng, n=cfg["n_seqs"], total=cfg["total"], lo=cfg["lo"], hi=cfg["hi"])
        cu = np.zeros(len(lens) + 1, dtype=np.int32)
        cu[1:] = np.cumsum(lens)
        t = int(cu[-1])
        h, d = cfg["heads"], cfg["head_dim"]
        q = _draw_bf16(rng, (t, h, d), 1.0)
        k = _draw_bf16(rng, (t, h, d), 1.0)
        v = _draw_bf16(rng, (t, h, d), 1.0)
        return AttnInputs(name=name, q=q, k=k, v=v, scale=_fp32_scale(d), causal=cfg["causal"],
                          cu_seqlens=cu, seed=seed)
    return random_inputs(seed, cfg["batch"], cfg["seqlen"], cfg["heads"], cfg["head_dim"],
                         cfg["causal"], q_std=cfg.get("q_std", 1.0),
                         with_do=cfg.get("with_do", False), name=name)
