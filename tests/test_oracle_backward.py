"""Pins for the oracle's backward (CPU only): finite differences of the oracle's
own forward, torch float64 autograd, and exact identities of the gradient."""
import math

import numpy as np
import pytest
import torch

from oracle import attention as A
from tiled_exact_attention_bf16_amd import inputs as I


def _rand(shape, seed, std=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * std


def _loss(q, k, v, do, scale, causal):
    o, _ = A.head_forward(q, k, v, scale, causal)
    return float((o * do).sum())


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("n,d", [(1, 2), (5, 3), (8, 4)])
def test_central_finite_differences(causal, n, d):
    q, k, v, do = (_rand((n, d), s) for s in (50 + n, 51 + n, 52 + n, 53 + n))
    scale = 0.7
    dq, dk, dv = A.head_backward(q, k, v, do, scale, causal)
    h = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(*x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args = {"q": q, "k": k, "v": v}
            args[name] = xp
            fp = _loss(args["q"], args["k"], args["v"], do, scale, causal)
            args[name] = xm
            fm = _loss(args["q"], args["k"], args["v"], do, scale, causal)
            num[idx] = (fp - fm) / (2 * h)
        assert np.max(np.abs(num - g)) <= 1e-8, name


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("n,d", [(17, 8), (64, 32)])
def test_against_torch_autograd_float64(causal, n, d):
    q, k, v, do = (_rand((n, d), s) for s in (60, 61, 62, 63))
    scale = 1.0 / math.sqrt(d)
    dq, dk, dv = A.head_backward(q, k, v, do, scale, causal)
    tq, tk, tv = (torch.from_numpy(x).clone().requires_grad_(True) for x in (q, k, v))
    s = scale * (tq @ tk.T)
    if causal:
        s = s.masked_fill(torch.triu(torch.ones(n, n, dtype=torch.bool), 1), float("-inf"))
    o = torch.softmax(s, dim=1) @ tv
    o.backward(torch.from_numpy(do))
    for mine, ref in ((dq, tq.grad), (dk, tk.grad), (dv, tv.grad)):
        assert np.max(np.abs(mine - ref.numpy())) <= 1e-11


@pytest.mark.parametrize("causal", [False, True])
def test_gradient_identities(causal):
    n, d = 48, 16
    q, k, v, do = (_rand((n, d), s, 2.0) for s in (70, 71, 72, 73))
    dq, dk, dv = A.head_backward(q, k, v, do, 0.3, causal)
    # rows of dS sum to zero, so the key gradients sum to zero
    assert np.max(np.abs(dk.sum(axis=0))) <= 1e-10
    # rows of P sum to one, so the value gradients sum to the output gradients
    assert np.max(np.abs(dv.sum(axis=0) - do.sum(axis=0))) <= 1e-10


def test_value_gradient_closed_form_single_key():
    # one key: P = 1, so dV_0 = sum_i dO_i and dQ = dK = 0
    q, k, v, do = _rand((6, 4), 80), _rand((1, 4), 81), _rand((1, 4), 82), _rand((6, 4), 83)
    dq, dk, dv = A.head_backward(q, k, v, do, 0.5, causal=False)
    assert np.allclose(dv[0], do.sum(axis=0), atol=1e-14)
    assert np.max(np.abs(dq)) <= 1e-14 and np.max(np.abs(dk)) <= 1e-14


def test_varlen_packing_invariance():
    inp = I.random_varlen_inputs(84, [7, 1, 12], heads=2, head_dim=8, causal=True, with_do=True)
    q, k, v, do = (I.bf16_bits_to_f64(t) for t in (inp.q, inp.k, inp.v, inp.do))
    dq, dk, dv = A.backward(q, k, v, do, inp.scale, True, cu_seqlens=inp.cu_seqlens)
    cu = inp.cu_seqlens
    for b in range(3):
        s0, s1 = int(cu[b]), int(cu[b + 1])
        g = A.backward(q[None, s0:s1], k[None, s0:s1], v[None, s0:s1], do[None, s0:s1], inp.scale, True)
        for full, part in zip((dq, dk, dv), g):
            assert np.array_equal(full[s0:s1], part[0])


@pytest.mark.parametrize("lq,lk", [(9, 40), (40, 9), (1, 17)])
def test_bottom_right_causal_against_torch_autograd(lq, lk):
    """Unequal lengths under the causal mask: torch's lower-right causal bias with
    float64 autograd (rows that see no key contribute nothing)."""
    from torch.nn.attention.bias import causal_lower_right
    d = 8
    q, do = _rand((lq, d), 70), _rand((lq, d), 71)
    k, v = _rand((lk, d), 72), _rand((lk, d), 73)
    scale = 1.0 / math.sqrt(d)
    dq, dk, dv = A.head_backward(q, k, v, do, scale, True)
    seen = np.arange(lq) + lk - lq >= 0
    tq, tk, tv = (torch.from_numpy(x).clone().requires_grad_(True) for x in (q, k, v))
    o = torch.nn.functional.scaled_dot_product_attention(tq[None, None], tk[None, None], tv[None, None],
                                                         attn_mask=causal_lower_right(lq, lk), scale=scale)[0, 0]
    o = torch.where(torch.from_numpy(seen)[:, None], o, torch.zeros_like(o))   # torch gives NaN rows there
    o.backward(torch.from_numpy(do))
    assert np.all(dq[~seen] == 0.0)
    for mine, ref in ((dq, tq.grad), (dk, tk.grad), (dv, tv.grad)):
        assert np.max(np.abs(mine - np.nan_to_num(ref.numpy()))) <= 1e-11


def test_given_output_enters_only_through_d():
    """The backward may be handed the forward output (rounded, as a kernel stores it):
    with the exact output nothing changes; a perturbation of O changes D_i by
    dD_i = dO_i . delta_i, which moves dQ_i by -scale * dD_i * sum_j P_ij k_j and dK_j
    by -scale * sum_i P_ij dD_i q_i, and leaves dV unchanged."""
    n, d = 40, 8
    q, k, v, do = (_rand((n, d), s) for s in (80, 81, 82, 83))
    base = A.head_backward(q, k, v, do, 0.4, True)
    o, _ = A.head_forward(q, k, v, 0.4, True)
    same = A.head_backward(q, k, v, do, 0.4, True, o=o)
    for x, y in zip(base, same):
        assert np.max(np.abs(x - y)) == 0.0
    delta = _rand((n, d), 84) * 1e-3
    dq2, dk2, dv2 = A.head_backward(q, k, v, do, 0.4, True, o=o + delta)
    dd = (do * delta).sum(axis=1)                       # change of D_i
    p = A.head_probabilities(q, k, 0.4, True)
    assert np.max(np.abs(dv2 - base[2])) == 0.0
    assert np.max(np.abs(dq2 - (base[0] - 0.4 * (p * dd[:, None]) @ k))) <= 1e-13
    assert np.max(np.abs(dk2 - (base[1] - 0.4 * (p * dd[:, None]).T @ q))) <= 1e-13
