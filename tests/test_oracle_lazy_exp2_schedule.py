"""Pins for the oracle's streaming model (lazy rescaling), the exp2 split model
and the longest-first ordering (CPU only)."""
import json
import math
import os

import numpy as np
import pytest

from oracle import attention as A
from oracle import exp2_split as E
from oracle import online_softmax as OS
from oracle import schedule as SCH

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_figures.json")))


def _rand(shape, seed, std=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * std


# --- lazy rescaling -------------------------------------------------------------

def test_reference_shift_cancels_in_closed_form():
    # sum_j 2^(x_j - m) v_j / sum_j 2^(x_j - m) does not depend on m
    x, v = _rand(50, 90, 4.0), _rand((50, 3), 91)
    outs = [(np.exp2(x - m)[:, None] * v).sum(0) / np.exp2(x - m).sum() for m in (-5.0, 0.0, x.max(), 30.0)]
    for o in outs[1:]:
        assert np.allclose(o, outs[0], rtol=0, atol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("reverse", [False, True])
def test_lazy_equals_eager_equals_definition(causal, reverse):
    thr = GOLDEN["lazy_rescale"]["threshold_log2"]
    q, k, v = _rand((96, 32), 92, 3.0), _rand((96, 32), 93), _rand((96, 32), 94)
    scale = 1 / math.sqrt(32)
    o_ref, lse_ref = A.head_forward(q, k, v, scale, causal)
    o8, lse8, st8 = OS.tiled_head_forward(q, k, v, scale, causal, 16, thr, reverse_tiles=reverse)
    o0, lse0, st0 = OS.tiled_head_forward(q, k, v, scale, causal, 16, 0.0, reverse_tiles=reverse)
    for o, lse in ((o8, lse8), (o0, lse0)):
        assert np.max(np.abs(o - o_ref)) <= 1e-13
        assert np.max(np.abs(lse - lse_ref)) <= 1e-12
    # laziness: fewer reference moves, weights bounded by 2^threshold (the page's factor)
    assert st8.rescales < st0.rescales
    assert st8.max_weight <= GOLDEN["lazy_rescale"]["threshold_factor"]
    assert st0.max_weight <= 1.0
    assert 2 ** thr == GOLDEN["lazy_rescale"]["threshold_factor"]


def test_lazy_in_fp32_stays_within_fp32_rounding():
    q, k, v = _rand((64, 64), 95, 3.0), _rand((256, 64), 96), _rand((256, 64), 97)
    scale = 0.125
    o_ref, lse_ref = A.head_forward(q, k, v, scale, False)
    o8, lse8, _ = OS.tiled_head_forward(q, k, v, scale, False, 32, 8.0, dtype=np.float32)
    assert np.max(np.abs(o8 - o_ref)) <= 2e-5
    assert np.max(np.abs(lse8 - lse_ref)) <= 2e-5


# --- exp2 split -------------------------------------------------------------------

def test_cubic_fit_properties():
    c = E.fit_cubic()
    assert c[0] == 1.0 and len(c) == GOLDEN["software_exp2"]["polynomial_degree"] + 1
    f = np.linspace(0, 1, 100001)
    p = c[0] + f * (c[1] + f * (c[2] + f * c[3]))
    rel = np.max(np.abs(p / np.exp2(f) - 1))
    # a cubic minimax fit of 2^f reaches ~8.6e-5; any dropped or wrong term is far worse
    assert rel < 1.0e-4
    assert rel > 5e-5


def test_exp2_split_special_values():
    xs = np.arange(-126, 9, dtype=np.float32)
    assert np.array_equal(E.exp2_split(xs), np.exp2(xs.astype(np.float64)).astype(np.float32))
    assert E.exp2_split(np.array([-np.inf, -127.5, -1000.0], dtype=np.float32)).tolist() == [0.0, 0.0, 0.0]


def test_exp2_split_within_one_bf16_ulp_on_dense_sweep():
    g = GOLDEN["software_exp2"]
    # every 61st fp32 bit pattern of [-126, 0) and of [0, 8]
    neg_bits = int(np.array(-126.0, dtype=np.float32).view(np.uint32))
    neg = np.arange(neg_bits, 0x80000000, -61, dtype=np.int64).astype(np.uint32).view(np.float32)
    assert neg[0] == -126.0 and neg[-1] < 0 and len(neg) > 1e7
    pos = np.arange(0, np.float32(8.0).view(np.uint32) + 1, 61, dtype=np.uint32).view(np.float32)
    grid = np.linspace(-126.0, 8.0, 1 << 22, dtype=np.float32)
    for xs in (neg, pos, grid):
        mine = E.exp2_split(xs)
        ref = np.exp2(xs.astype(np.float64)).astype(np.float32)
        ulp = E.bf16_ulp_distance(mine, ref)
        assert np.mean(ulp <= g["max_bf16_ulp"]) >= g["fraction_of_inputs"]
        assert np.mean(ulp == 0) >= 0.985


# --- longest-first schedule --------------------------------------------------------

@pytest.mark.parametrize("causal", [False, True])
def test_item_cost_matches_brute_force(causal):
    for length in (1, 5, 64, 100, 129, 300):
        for bm, bn in ((64, 64), (128, 64), (256, 128)):
            for b0 in range(0, length, bm):
                tiles = set()
                for i in range(b0, min(b0 + bm, length)):
                    for j in range(length):
                        if not causal or j <= i:
                            tiles.add(j // bn)
                assert SCH.item_cost(b0, bm, length, length, bn, causal) == len(tiles)


def test_longest_first_order_validity():
    items = SCH.work_items([300, 5, 1000, 129], 128, 64, causal=True)
    order = SCH.longest_first(items)
    assert SCH.is_longest_first(order, items)
    assert not SCH.is_longest_first(items, items)          # natural order increases cost
    assert not SCH.is_longest_first(order[:-1], items)     # an item is missing


def test_grouped_order_hand_example():
    # causal, 128-row items against 64-key tiles: lengths 300 and 1000 give costs
    # (2, 4, 5) and (2, 4, 6, ..., 16); buckets of width 4 (two items' growth)
    items = SCH.work_items([300, 1000], 128, 64, causal=True)
    assert SCH.bucket_width(128, 64, group=2) == 4
    order = SCH.grouped_longest_first(items, 4)
    assert [(b, t) for b, t, _ in order] == [(1, 7), (1, 6), (1, 5), (1, 4), (1, 3),
                                             (0, 2), (0, 1), (1, 2), (1, 1), (0, 0), (1, 0)]
    assert SCH.is_grouped_longest_first(order, items, 4)
    # the other sequence's run first inside a bucket is as valid
    alt = order[:5] + order[7:9] + order[5:7] + order[9:]
    assert SCH.is_grouped_longest_first(alt, items, 4)


def test_grouped_order_rejections():
    items = SCH.work_items([300, 1000], 128, 64, causal=True)
    cost = {(b, t): c for b, t, c in items}
    mk = lambda bt: [(b, t, cost[(b, t)]) for b, t in bt]
    good = [(1, 7), (1, 6), (1, 5), (1, 4), (1, 3), (0, 2), (0, 1), (1, 2), (1, 1), (0, 0), (1, 0)]
    assert SCH.is_grouped_longest_first(mk(good), items, 4)
    # sequence 0's run in bucket 1 interrupted by sequence 1
    split = good[:5] + [(0, 2), (1, 2), (0, 1), (1, 1)] + good[9:]
    assert not SCH.is_grouped_longest_first(mk(split), items, 4)
    # cost rising inside a run (12 before 14 in bucket 3)
    rising = good[:1] + [(1, 5), (1, 6)] + good[3:]
    assert not SCH.is_grouped_longest_first(mk(rising), items, 4)
    # the most expensive bucket last
    assert not SCH.is_grouped_longest_first(mk(good[1:] + good[:1]), items, 4)
    assert not SCH.is_grouped_longest_first(mk(good[:-1]), items, 4)   # an item missing
    assert not SCH.is_grouped_longest_first(items, items, 4)           # natural order
    # with wider buckets the strict longest-first order interleaves the sequences
    many = SCH.work_items([300, 5, 1000, 129, 700], 128, 64, causal=True)
    assert not SCH.is_grouped_longest_first(SCH.longest_first(many), many, 8)


def test_grouped_order_is_valid_for_random_lengths():
    import random
    rnd = random.Random(3)
    for _ in range(50):
        lens = [rnd.randint(1, 3000) for _ in range(rnd.randint(1, 9))]
        for causal in (False, True):
            items = SCH.work_items(lens, 256, 64, causal)
            w = SCH.bucket_width(256, 64)
            order = SCH.grouped_longest_first(items, w)
            assert SCH.is_grouped_longest_first(order, items, w)
            # bucket order refines the strict one: costs never rise by a bucket or more
            costs = [c for _, _, c in order]
            assert all(b - a < w for a, b in zip(costs, costs[1:]) if b > a)
