"""Input generators (determinism, bf16 narrowing) and the FLOP convention (CPU only)."""
import json
import math
import os

import numpy as np

from tiled_exact_attention_bf16_amd import inputs as I
from tiled_exact_attention_bf16_amd import workload as W

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_figures.json")))


def test_bf16_narrowing_round_to_nearest_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 0.0, 3.0e38, 1.0 + 2 ** -8 + 2 ** -20],
                 dtype=np.float32)
    bits = I.f32_to_bf16_bits(x)
    assert bits.tolist() == [0x3F80, 0x3F80, 0x3F82, 0xC020, 0x0000, 0x7F62, 0x3F81]
    assert np.array_equal(I.bf16_bits_to_f32(bits[:5]), np.array([1.0, 1.0, 1.0 + 2 ** -6, -2.5, 0.0],
                                                                 dtype=np.float32))


def test_generators_are_deterministic():
    a = I.random_inputs(7, 2, 33, 3, 64, causal=True, with_do=True)
    b = I.random_inputs(7, 2, 33, 3, 64, causal=True, with_do=True)
    for t in ("q", "k", "v", "do"):
        assert np.array_equal(getattr(a, t), getattr(b, t))
    c = I.random_inputs(8, 2, 33, 3, 64, causal=True)
    assert not np.array_equal(a.q, c.q)


def test_varlen_recipe_for_the_packed_workload():
    for seed in (0, 1, 2, 4):
        lens = I.varlen_lengths(np.random.default_rng(seed), n=32, total=131072, lo=128, hi=16384)
        assert lens.sum() == 131072 and len(lens) == 32
        assert lens.min() >= 128 and lens.max() <= 16384


def test_q_std_scales_the_query_draws():
    a = I.random_inputs(3, 1, 512, 2, 64, causal=True, q_std=3.0)
    q = I.bf16_bits_to_f64(a.q)
    k = I.bf16_bits_to_f64(a.k)
    assert 2.9 < q.std() < 3.1 and 0.95 < k.std() < 1.05


def test_flop_convention_matches_the_pages_tile_roofline():
    g = GOLDEN["roofline_tile"]
    bm, bn, d = g["tile_q"], g["tile_k"], g["head_dim"]
    fwd = W.fwd_flops([bm], [bn], 1, d, causal=False)
    bwd = W.bwd_flops([bm], [bn], 1, d, causal=False)
    assert fwd / g["bf16_tensor_ops_per_clk_per_sm"] == g["fwd_mma_cycles"]
    assert bwd / g["bf16_tensor_ops_per_clk_per_sm"] == g["bwd_mma_cycles"]
    # one exponential per visible pair
    assert W.visible_pairs(bm, bn, False) / g["exp_ops_per_clk_per_sm"] == g["fwd_exp_cycles"]


def test_causal_pair_count():
    for n in (1, 2, 7, 128, 8192):
        brute = sum(i + 1 for i in range(n)) if n < 10000 else None
        assert W.visible_pairs(n, n, True) == brute
    assert W.visible_pairs(8192, 8192, True) * 2 - 8192 == 8192 * 8192
    # unequal lengths under the causal mask: brute force over the bottom-right rule
    for lq, lk in ((1, 9), (9, 1), (5, 12), (12, 5), (7, 7), (3, 1000)):
        brute = sum(1 for i in range(lq) for j in range(lk) if j <= i + lk - lq)
        assert W.visible_pairs(lq, lk, True) == brute
    # the headline shape: B=2, H=16, S=8192, d=128 causal
    assert W.fwd_flops([8192] * 2, [8192] * 2, 16, 128, True) == 4 * 128 * 16 * 2 * 8192 * 8193 // 2
    assert math.isclose(W.fwd_flops([8192] * 2, [8192] * 2, 16, 128, True), 5.498e11, rel_tol=1e-3)
