"""Pins for the oracle's forward (CPU only).

Each check ties oracle.attention to something other than itself: closed forms,
invariants of softmax attention, brute-force loops on tiny inputs, and
torch's float64 attention as an independent library routine.
"""
import math

import numpy as np
import pytest
import torch

from oracle import attention as A
from tiled_exact_attention_bf16_amd import inputs as I


def _rand(shape, seed, std=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * std


# --- the definition: rows of P are positive and sum to one -------------------

@pytest.mark.parametrize("causal", [False, True])
def test_softmax_rows_sum_to_one(causal):
    q, k = _rand((37, 16), 1), _rand((37, 16), 2)
    p = A.head_probabilities(q, k, 0.25, causal)
    assert np.all(p >= 0)
    assert np.max(np.abs(p.sum(axis=1) - 1.0)) <= 1e-12
    if causal:
        assert np.all(np.triu(p, 1) == 0.0)
        assert np.all(p[np.tril_indices(37)] > 0)


# --- closed-form special cases -------------------------------------------------

def test_single_key():
    q, k, v = _rand((9, 8), 3), _rand((1, 8), 4), _rand((1, 8), 5)
    o, lse = A.head_forward(q, k, v, 0.3, causal=False)
    assert np.array_equal(o, np.repeat(v, 9, axis=0))
    assert np.allclose(lse, 0.3 * (q @ k[0]), rtol=0, atol=1e-14)


def test_causal_row_zero_copies_first_value():
    q, k, v = _rand((12, 8), 6), _rand((12, 8), 7), _rand((12, 8), 8)
    o, lse = A.head_forward(q, k, v, 0.5, causal=True)
    assert np.array_equal(o[0], v[0])
    assert lse[0] == pytest.approx(0.5 * float(q[0] @ k[0]), abs=1e-14)


@pytest.mark.parametrize("causal", [False, True])
def test_zero_query_averages_visible_values(causal):
    n = 10
    q, k, v = np.zeros((n, 8)), _rand((n, 8), 9), _rand((n, 8), 10)
    o, lse = A.head_forward(q, k, v, 0.7, causal)
    for i in range(n):
        vis = i + 1 if causal else n
        assert np.allclose(o[i], v[:vis].mean(axis=0), atol=1e-14)
        assert lse[i] == pytest.approx(math.log(vis), abs=1e-14)


def test_identical_keys_and_zero_scale_are_uniform():
    q, v = _rand((6, 8), 11), _rand((6, 8), 12)
    k_same = np.repeat(_rand((1, 8), 13), 6, axis=0)
    o, _ = A.head_forward(q, k_same, v, 0.9, causal=False)
    assert np.allclose(o, v.mean(axis=0)[None, :], atol=1e-14)
    o0, lse0 = A.head_forward(q, _rand((6, 8), 14), v, 0.0, causal=False)
    assert np.allclose(o0, v.mean(axis=0)[None, :], atol=1e-14)
    assert np.allclose(lse0, math.log(6), atol=1e-14)


def test_dominant_logit_selects_its_value():
    k = np.eye(8)
    v = _rand((8, 8), 15)
    q = 1000.0 * np.eye(8)[[3, 5]]
    o, lse = A.head_forward(q, k, v, 1.0, causal=False)
    assert np.allclose(o[0], v[3], atol=1e-12) and np.allclose(o[1], v[5], atol=1e-12)
    assert np.allclose(lse, 1000.0, atol=1e-12)


# --- invariants ------------------------------------------------------------------

@pytest.mark.parametrize("causal", [False, True])
def test_lse_bounds_and_convex_hull(causal):
    q, k, v = _rand((40, 16), 16, 3.0), _rand((40, 16), 17), _rand((40, 16), 18)
    scale = 0.25
    o, lse = A.head_forward(q, k, v, scale, causal)
    s = scale * q @ k.T
    for i in range(40):
        vis = i + 1 if causal else 40
        mx = s[i, :vis].max()
        assert mx - 1e-12 <= lse[i] <= mx + math.log(vis) + 1e-12
        assert np.all(o[i] >= v[:vis].min(axis=0) - 1e-12)
        assert np.all(o[i] <= v[:vis].max(axis=0) + 1e-12)


def test_key_permutation_invariance_and_query_equivariance():
    q, k, v = _rand((20, 8), 19), _rand((31, 8), 20), _rand((31, 8), 21)
    o, lse = A.head_forward(q, k, v, 0.4, causal=False)
    pk = np.random.default_rng(22).permutation(31)
    o2, lse2 = A.head_forward(q, k[pk], v[pk], 0.4, causal=False)
    assert np.allclose(o, o2, atol=1e-13) and np.allclose(lse, lse2, atol=1e-13)
    pq = np.random.default_rng(23).permutation(20)
    o3, lse3 = A.head_forward(q[pq], k, v, 0.4, causal=False)
    assert np.allclose(o3, o[pq], atol=1e-13) and np.allclose(lse3, lse[pq], atol=1e-13)


def test_row_subset_and_row_blocking_do_not_change_results(monkeypatch):
    q, k, v = _rand((50, 8), 24), _rand((50, 8), 25), _rand((50, 8), 26)
    o, lse = A.head_forward(q, k, v, 0.3, causal=True)
    rows = [0, 7, 31, 49]
    o_r, lse_r = A.head_forward(q, k, v, 0.3, causal=True, rows=rows)
    assert np.array_equal(o_r, o[rows]) and np.array_equal(lse_r, lse[rows])
    monkeypatch.setattr(A, "ROW_BLOCK", 3)
    o_b, lse_b = A.head_forward(q, k, v, 0.3, causal=True)
    assert np.allclose(o_b, o, atol=1e-14) and np.allclose(lse_b, lse, atol=1e-14)


def test_packing_invariance_and_head_independence():
    inp = I.random_varlen_inputs(27, [5, 0, 17, 1, 9], heads=3, head_dim=8, causal=True)
    q, k, v = (I.bf16_bits_to_f64(t) for t in (inp.q, inp.k, inp.v))
    o, lse = A.forward(q, k, v, inp.scale, True, cu_seqlens=inp.cu_seqlens)
    cu = inp.cu_seqlens
    for b in range(5):
        s0, s1 = int(cu[b]), int(cu[b + 1])
        ob, lseb = A.forward(q[None, s0:s1], k[None, s0:s1], v[None, s0:s1], inp.scale, True)
        assert np.array_equal(o[s0:s1], ob[0])
        assert np.array_equal(lse[:, s0:s1], lseb[0])
    # one head alone equals the slice of the full result
    o1, lse1 = A.forward(q, k, v, inp.scale, True, cu_seqlens=cu, heads=[1])
    assert np.array_equal(o1[:, 1], o[:, 1]) and np.array_equal(lse1[1], lse[1])


def test_no_visible_key_gives_zero_output_and_minus_inf_lse():
    q = _rand((4, 8), 28)
    o, lse = A.head_forward(q, np.zeros((0, 8)), np.zeros((0, 8)), 0.5, causal=False)
    assert np.all(o == 0) and np.all(np.isneginf(lse))


# --- brute force on tiny shapes (pure Python loops) --------------------------------

@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("n,d", [(1, 1), (3, 2), (8, 4)])
def test_brute_force_loops(causal, n, d):
    q, k, v = _rand((n, d), 29 + n), _rand((n, d), 30 + n), _rand((n, d), 31 + n)
    scale = 0.6
    o, lse = A.head_forward(q, k, v, scale, causal)
    for i in range(n):
        scores = []
        for j in range(n):
            if causal and j > i:
                continue
            scores.append((j, scale * sum(q[i, t] * k[j, t] for t in range(d))))
        mx = max(s for _, s in scores)
        w = [(j, math.exp(s - mx)) for j, s in scores]
        tot = sum(x for _, x in w)
        for t in range(d):
            ref = sum(x * v[j, t] for j, x in w) / tot
            assert abs(o[i, t] - ref) <= 1e-13
        assert abs(lse[i] - (mx + math.log(tot))) <= 1e-13


# --- torch float64 attention as an independent library routine ---------------------

@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("lq,lk,d", [(33, 33, 16), (64, 64, 64), (5, 70, 8)])
def test_against_torch_float64(causal, lq, lk, d):
    if causal and lq != lk:
        pytest.skip("rectangular causal: see test_bottom_right_causal_against_torch")
    q, k, v = _rand((lq, d), 40, 2.0), _rand((lk, d), 41), _rand((lk, d), 42)
    scale = 1.0 / math.sqrt(d)
    o, lse = A.head_forward(q, k, v, scale, causal)
    tq, tk, tv = (torch.from_numpy(x)[None, None] for x in (q, k, v))
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, scale=scale)
    assert np.max(np.abs(o - ref[0, 0].numpy())) <= 1e-12
    s = scale * (torch.from_numpy(q) @ torch.from_numpy(k).T)
    if causal:
        s = s.masked_fill(torch.triu(torch.ones(lq, lk, dtype=torch.bool), 1), float("-inf"))
    assert np.max(np.abs(lse - torch.logsumexp(s, dim=1).numpy())) <= 1e-12


# --- causal with unequal query and key lengths (bottom-right alignment) ------------

@pytest.mark.parametrize("lq,lk,d", [(5, 70, 8), (1, 33, 16), (17, 64, 32), (64, 17, 8), (2, 1, 4)])
def test_bottom_right_causal_against_torch(lq, lk, d):
    """torch's lower-right causal bias is an independent implementation of the
    alignment (the last query sees every key)."""
    from torch.nn.attention.bias import causal_lower_right
    q, k, v = _rand((lq, d), 50, 2.0), _rand((lk, d), 51), _rand((lk, d), 52)
    scale = 1.0 / math.sqrt(d)
    o, lse = A.head_forward(q, k, v, scale, True)
    seen = np.isfinite(lse)
    assert np.all(seen == (np.arange(lq) + lk - lq >= 0))
    assert np.all(o[~seen] == 0.0)
    tq, tk, tv = (torch.from_numpy(x)[None, None] for x in (q, k, v))
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=causal_lower_right(lq, lk),
                                                           scale=scale)[0, 0].numpy()
    assert np.max(np.abs(o[seen] - ref[seen])) <= 1e-12


@pytest.mark.parametrize("lq,lk", [(7, 40), (40, 7), (1, 9)])
def test_bottom_right_causal_is_the_tail_of_the_square_problem(lq, lk):
    """With Lq < Lk the queries behave as the last Lq of Lk positions; with Lq > Lk
    the last Lk queries behave as a square problem and the others see nothing."""
    d = 8
    k, v = _rand((lk, d), 60), _rand((lk, d), 61)
    if lq <= lk:
        full_q = _rand((lk, d), 62)
        q = full_q[lk - lq:]
        o_sq, lse_sq = A.head_forward(full_q, k, v, 0.7, True)
        o, lse = A.head_forward(q, k, v, 0.7, True)
        assert np.max(np.abs(o - o_sq[lk - lq:])) <= 1e-13 and np.max(np.abs(lse - lse_sq[lk - lq:])) <= 1e-13
    else:
        q = _rand((lq, d), 63)
        o, lse = A.head_forward(q, k, v, 0.7, True)
        o_sq, lse_sq = A.head_forward(q[lq - lk:], k, v, 0.7, True)
        assert np.all(o[:lq - lk] == 0.0) and np.all(np.isneginf(lse[:lq - lk]))
        assert np.max(np.abs(o[lq - lk:] - o_sq)) <= 1e-13 and np.max(np.abs(lse[lq - lk:] - lse_sq)) <= 1e-13
