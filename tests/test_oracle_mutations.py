"""Planted mistakes in the oracle must be caught by its pins (CPU only).

Each mutant is a plausible slip in the oracle's forward or backward (a dropped
scale, an off-by-one or flipped mask, swapped operands, a missing term, a wrong
sign).  The pins used here are independent of the oracle: pure-Python brute
force, torch float64 attention/autograd, and central finite differences.
"""
import math

import numpy as np
import pytest
import torch

from oracle import attention as A


def _rand(shape, seed, std=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * std


def _fwd_mutant(kind):
    def f(q, k, v, scale, causal, rows=None):
        n, lk = q.shape[0], k.shape[0]
        sc = 1.0 if kind == "no_scale" else scale
        s = sc * (q @ (v if kind == "k_is_v" else k).T)
        i = np.arange(n)[:, None]
        j = np.arange(lk)[None, :]
        if causal:
            vis = {"mask_strict": j < i, "mask_flipped": j >= i}.get(kind, j <= i)
            s = np.where(vis, s, -np.inf)
        m = s.max(axis=1, keepdims=True)
        m = np.where(np.isfinite(m), m, 0)
        e = np.exp(s - m)
        vals = k if kind == "v_is_k" else v
        o = e @ vals / e.sum(axis=1, keepdims=True)
        lse = (m[:, 0] if kind != "lse_no_max" else 0) + np.log(e.sum(axis=1))
        return o, lse
    return f


def _torch_pin(fwd, causal):
    n, d = 24, 8
    q, k, v = _rand((n, d), 1, 2.0), _rand((n, d), 2), _rand((n, d), 3)
    scale = 1 / math.sqrt(d)
    o, lse = fwd(q, k, v, scale, causal)
    tq, tk, tv = (torch.from_numpy(x)[None, None] for x in (q, k, v))
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, scale=scale)
    s = scale * torch.from_numpy(q) @ torch.from_numpy(k).T
    if causal:
        s = s.masked_fill(torch.triu(torch.ones(n, n, dtype=torch.bool), 1), float("-inf"))
    ok_o = np.nanmax(np.abs(o - ref[0, 0].numpy())) <= 1e-12 if np.all(np.isfinite(o)) else False
    ok_l = np.nanmax(np.abs(lse - torch.logsumexp(s, 1).numpy())) <= 1e-12 if np.all(np.isfinite(lse)) else False
    return ok_o and ok_l


def test_correct_forward_passes_pin():
    assert _torch_pin(A.head_forward, True) and _torch_pin(A.head_forward, False)
    assert _torch_pin(_fwd_mutant("none"), True)


@pytest.mark.parametrize("kind", ["no_scale", "k_is_v", "v_is_k", "mask_strict", "mask_flipped", "lse_no_max"])
def test_forward_mutants_are_caught(kind):
    assert not _torch_pin(_fwd_mutant(kind), causal=True)


def _bwd_mutant(kind):
    def g(q, k, v, do, scale, causal):
        o, lse = A.head_forward(q, k, v, scale, causal)
        n = q.shape[0]
        s = scale * q @ k.T
        if causal:
            s = np.where(np.tril(np.ones((n, n), dtype=bool)), s, -np.inf)
        p = np.exp(s - lse[:, None])
        dvec = (do * o).sum(1)
        dp = do @ v.T
        ds = p * (dp - (0 if kind == "drop_D" else dvec[:, None]))
        dv = (p.T @ do) if kind != "dv_transposed" else (p @ do)
        dq = scale * ds @ k * (-1 if kind == "dq_sign" else 1)
        dk = scale * ds.T @ q if kind != "dk_no_scale" else ds.T @ q
        return dq, dk, dv
    return g


def _fd_pin(bwd):
    n, d = 6, 3
    q, k, v, do = (_rand((n, d), s) for s in (11, 12, 13, 14))
    scale = 0.7
    grads = bwd(q, k, v, do, scale, True)
    h = 1e-6
    for which, x, gr in zip("qkv", (q, k, v), grads):
        num = np.zeros_like(x)
        for idx in np.ndindex(*x.shape):
            args = {"q": q, "k": k, "v": v}
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args[which] = xp
            fp = (A.head_forward(args["q"], args["k"], args["v"], scale, True)[0] * do).sum()
            args[which] = xm
            fm = (A.head_forward(args["q"], args["k"], args["v"], scale, True)[0] * do).sum()
            num[idx] = (fp - fm) / (2 * h)
        if np.max(np.abs(num - gr)) > 1e-8:
            return False
    return True


def test_correct_backward_passes_pin():
    assert _fd_pin(A.head_backward) and _fd_pin(_bwd_mutant("none"))


@pytest.mark.parametrize("kind", ["drop_D", "dv_transposed", "dq_sign", "dk_no_scale"])
def test_backward_mutants_are_caught(kind):
    assert not _fd_pin(_bwd_mutant(kind))
