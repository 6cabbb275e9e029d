"""Forward parity: the HIP path (through the C ABI) against the fp64 oracle."""
import numpy as np
import pytest
import torch

from oracle import schedule as OS
from tiled_exact_attention_bf16_amd import inputs as I
from tests.gpu_util import (TOL_LSE, TOL_MAX, TOL_MEAN, bf16_rounding_floor, errors, gpu_head, gpu_lse_head,
                            lse_error, named_inputs, oracle_fwd_head, oracle_map, say, upload)

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from tiled_exact_attention_bf16_amd import attention as FA


def run_fwd(inp, tuning=None):
    q, k, v, _, cu = upload(inp)
    o, lse = FA.fwd(q, k, v, inp.scale, inp.causal, cu_seqlens_q=cu,
                    max_seqlen_q=inp.max_seqlen() if inp.varlen else None, tuning=tuning)
    torch.cuda.synchronize()
    return o, lse


def check_heads(inp, o, lse, pairs, rows=None, tag="", strict=False):
    """strict: the literal bar (named workloads); else mean-abs may add the bf16 output
    floor.  O must be finite; LSE must be finite where the oracle's is and exactly
    -inf where the row sees no key (lse_error counts anything else as infinite)."""
    worst = (0.0, 0.0, 0.0)
    refs = oracle_map(lambda bh: oracle_fwd_head(inp, bh[0], bh[1], rows=rows), pairs)
    for (b, h), (ref_o, ref_lse) in zip(pairs, refs):
        go, gl = gpu_head(o, inp, b, h), gpu_lse_head(lse, inp, b, h)
        if rows is not None:
            go, gl = go[rows], gl[rows]
        assert np.all(np.isfinite(go)), (tag, b, h)
        assert not np.isnan(gl).any(), (tag, b, h, "NaN LSE")
        mx, mean = errors(go, ref_o)
        le = lse_error(gl, ref_lse)
        worst = (max(worst[0], mx), max(worst[1], mean), max(worst[2], le))
        mean_bar = TOL_MEAN + (0.0 if strict else bf16_rounding_floor(ref_o))
        assert mx <= TOL_MAX and mean <= mean_bar and le <= TOL_LSE, (tag, b, h, mx, mean, le)
    say(f"[fwd {tag}] max-abs {worst[0]:.3e} mean-abs {worst[1]:.3e} lse {worst[2]:.3e}")
    return worst


def whole_tensor_sane(o, lse):
    """Checks over every element of a named workload's outputs (cheap, no oracle): O
    finite, LSE free of NaN (-inf only for rows that see no key, which none of the named
    workloads has)."""
    assert bool(torch.isfinite(o).all()), "non-finite O"
    assert bool(torch.isfinite(lse).all()), "non-finite LSE"


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("s", [1, 2, 17, 127, 128, 129, 255, 256, 1000])
def test_small_shapes(s, causal, d):
    inp = I.random_inputs(100 + s, 2, s, 3, d, causal)
    say(f"case s={s} causal={causal} d={d}")
    o, lse = run_fwd(inp)
    check_heads(inp, o, lse, [(b, h) for b in range(2) for h in range(3)], tag=f"s{s}c{int(causal)}d{d}")


@pytest.mark.parametrize("qt", [1, 2])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("lq,lk", [(1, 4096), (7, 1000), (128, 4096), (300, 257), (1000, 64), (64, 1000), (257, 300)])
def test_causal_unequal_lengths(lq, lk, d, qt):
    # bottom-right causal alignment; with lq > lk the first lq - lk rows see no key
    inp = I.random_inputs(300 + lq + lk, 2, lq, 2, d, True, seqlen_k=lk)
    say(f"case causal lq={lq} lk={lk} d={d} q_tiles={qt}")
    o, lse = run_fwd(inp, FA.Tuning(q_tiles_per_workgroup=qt, key_splits=1))
    check_heads(inp, o, lse, [(b, h) for b in range(2) for h in range(2)], tag=f"causal{lq}x{lk}d{d}qt{qt}")


# key splits: short query sequences against long key sequences (generation with a
# cache); each chunk's partial O and LSE are merged by LSE weights
@pytest.mark.parametrize("splits", [-1, 1, 3, 8])
@pytest.mark.parametrize("b,lq,lk,h,d,causal", [(4, 1, 8192, 8, 128, False), (4, 1, 8192, 8, 128, True),
                                               (2, 7, 5000, 4, 64, True), (1, 128, 16384, 4, 128, True),
                                               (2, 33, 3000, 4, 128, False), (1, 300, 4096, 2, 128, True)])
def test_key_splits(b, lq, lk, h, d, causal, splits):
    inp = I.random_inputs(500 + lq + lk, b, lq, h, d, causal, seqlen_k=lk)
    say(f"case split={splits} b={b} lq={lq} lk={lk} h={h} d={d} causal={causal}")
    o, lse = run_fwd(inp, FA.Tuning(key_splits=splits))
    pairs = [(0, 0), (b - 1, h - 1)]
    check_heads(inp, o, lse, pairs, tag=f"split{splits} {b}x{lq}x{lk}x{h}d{d}c{int(causal)}")


@pytest.mark.parametrize("splits", [-1, 4])
@pytest.mark.parametrize("causal", [False, True])
def test_key_splits_varlen_separate_key_lengths(causal, splits):
    q_lens = [1, 0, 5, 64, 130, 1, 17]
    k_lens = [3000, 7, 4100, 64, 2000, 0, 9000]
    inp = I.random_varlen_qk_inputs(77, q_lens, k_lens, heads=2, head_dim=128, causal=causal)
    say(f"case varlen q/k lengths split={splits} causal={causal}")
    q, k, v, _, cu = upload(inp)
    cu_k = torch.from_numpy(inp.cu_seqlens_k).cuda()
    o, lse = FA.fwd(q, k, v, inp.scale, causal, cu_seqlens_q=cu, cu_seqlens_k=cu_k, max_seqlen_q=inp.max_seqlen(),
                    max_seqlen_k=inp.max_seqlen_k(), tuning=FA.Tuning(key_splits=splits))
    torch.cuda.synchronize()
    check_heads(inp, o, lse, [(bb, hh) for bb in range(len(q_lens)) for hh in range(2)], tag=f"varlenqk split{splits}")


@pytest.mark.parametrize("variant", [(0, 8, 1), (0, 8, 2), (2, 8, 2), (4, 8, 2), (2, 8, 1), (0, 0, 2), (0, 0, 1)])
@pytest.mark.parametrize("causal", [False, True])
def test_variants_with_wide_logits(variant, causal):
    # Q ~ N(0, 3^2): row maxima grow across key tiles, so lazy rescales fire
    poly, tau, qt = variant
    inp = I.random_inputs(7, 1, 700, 4, 128, causal, q_std=3.0)
    say(f"case variant={variant} causal={causal}")
    o, lse = run_fwd(inp, FA.Tuning(poly, tau, qt))
    check_heads(inp, o, lse, [(0, h) for h in range(4)], tag=f"variant{variant}c{int(causal)}")


@pytest.mark.parametrize("qt", [1, 2])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
def test_varlen_ragged_with_empty_and_single(causal, d, qt):
    lens = [0, 1, 5, 128, 129, 300, 17, 0, 256, 511]
    inp = I.random_varlen_inputs(11, lens, heads=2, head_dim=d, causal=causal)
    say(f"case varlen causal={causal} d={d} q_tiles={qt}")
    o, lse = run_fwd(inp, FA.Tuning(q_tiles_per_workgroup=qt))
    check_heads(inp, o, lse, [(b, h) for b in range(len(lens)) for h in range(2)], tag=f"varlen{d}qt{qt}")


def test_config_c1_full():
    inp = named_inputs("c1")
    o, lse = run_fwd(inp)
    whole_tensor_sane(o, lse)
    check_heads(inp, o, lse, [(0, 0), (0, 1)], tag="c1", strict=True)


@pytest.mark.parametrize("name", ["c2", "c2_causal", "headline"])
def test_configs_every_head(name):
    # every (batch, head) pair, every row, against the oracle at the literal bar
    inp = named_inputs(name)
    say(f"case {name}: all {inp.batch * inp.num_heads} (batch, head) pairs")
    o, lse = run_fwd(inp)
    whole_tensor_sane(o, lse)
    check_heads(inp, o, lse, [(b, h) for b in range(inp.batch) for h in range(inp.num_heads)], tag=name,
                strict=True)


def test_config_c3_full_rows_and_every_head():
    inp = named_inputs("c3")
    say("case c3")
    o, lse = run_fwd(inp)
    whole_tensor_sane(o, lse)
    # three heads on every one of their 16,384 rows ...
    check_heads(inp, o, lse, [(0, 0), (0, 17), (0, 31)], tag="c3 full rows", strict=True)
    # ... and 256 rows (both ends and a seeded middle sample) of every other head
    rng = np.random.default_rng(33)
    rows = np.unique(np.r_[0:64, rng.choice(np.arange(64, 16384 - 64), 128, replace=False), 16384 - 64:16384])
    others = [(0, h) for h in range(inp.num_heads) if h not in (0, 17, 31)]
    check_heads(inp, o, lse, others, rows=rows, tag="c3 sampled rows", strict=True)


def test_config_c4_every_sequence():
    inp = named_inputs("c4")
    say("case c4")
    o, lse = run_fwd(inp)
    whole_tensor_sane(o, lse)
    lens = inp.seqlens()
    # every sequence on all of its rows for heads 0 and 15
    check_heads(inp, o, lse, [(b, h) for b in range(len(lens)) for h in (0, 15)], tag="c4 heads 0,15",
                strict=True)
    # every other head on the three shortest sequences and one of middle length
    order = np.argsort(lens, kind="stable")
    seqs = [int(b) for b in order[:3]] + [int(order[len(order) // 2])]
    check_heads(inp, o, lse, [(b, h) for b in seqs for h in range(1, 15)], tag="c4 other heads", strict=True)


def test_grouped_longest_first_schedule_c4():
    inp = named_inputs("c4")
    q, k, _, _, cu = upload(inp)
    for qt in (1, 2):
        tile_rows, order = FA.build_schedule(q, k, cu, True, max_seqlen=inp.max_seqlen(),
                                             tuning=FA.Tuning(q_tiles_per_workgroup=qt))
        lens = inp.seqlens()
        cost = {(b, t): OS.item_cost(t * tile_rows, tile_rows, int(lens[b]), int(lens[b]), 64, True)
                for b in range(len(lens)) for t in range(-(-int(lens[b]) // tile_rows))}
        items = [(b, t, c) for (b, t), c in cost.items()]
        got = [(b, t, cost[(b, t)]) for b, t in order]
        assert OS.is_grouped_longest_first(got, items, OS.bucket_width(tile_rows, 64))
        say(f"[schedule] tile_rows={tile_rows} items={len(order)} first cost {got[0][2]} last cost {got[-1][2]}")


def test_output_canaries_and_strided_views():
    inp = I.random_inputs(21, 2, 333, 3, 128, True)
    q, k, v, _, _ = upload(inp)
    # O written through a view that skips a guard head; LSE followed by a guard region
    o_big = torch.full((2, 333, 4, 128), float("nan"), dtype=torch.bfloat16, device="cuda")
    o_view = o_big[:, :, 1:, :]
    lse_big = torch.full((2 * 3 * 333 + 4096,), float("nan"), dtype=torch.float32, device="cuda")
    lse_view = lse_big[: 2 * 3 * 333].view(2, 3, 333)
    FA.fwd(q, k, v, inp.scale, True, out=o_view, lse=lse_view)
    torch.cuda.synchronize()
    assert bool(torch.isnan(o_big[:, :, 0]).all()), "write outside the strided output"
    assert bool(torch.isnan(lse_big[2 * 3 * 333:]).all()), "write past the LSE buffer"
    assert bool(torch.isfinite(o_view).all()) and bool(torch.isfinite(lse_view).all())
    check_heads(inp, o_view, lse_view, [(b, h) for b in range(2) for h in range(3)], tag="strided")


@pytest.mark.parametrize("case", ["fixed_full", "fixed_causal", "fixed_causal_d64", "varlen_causal", "key_split"])
def test_fp32_output_is_the_unrounded_output(case):
    """An fp32 O is the normalised output before its bf16 rounding: rounded to bf16 (RNE)
    it equals the bf16 O of the same call bit for bit, the LSE is the same, and it meets
    the bar against the oracle."""
    tuning = None
    if case == "varlen_causal":
        inp = I.random_varlen_inputs(911, [1, 300, 64, 0, 1000], 3, 128, True)
    elif case == "key_split":
        inp = I.random_inputs(913, 2, 7, 4, 128, True, seqlen_k=5000)
        tuning = FA.Tuning(key_splits=4)
    else:
        inp = I.random_inputs(917, 2, 700, 3, 64 if case.endswith("d64") else 128, case.startswith("fixed_causal"))
    say(f"case fp32 O {case}")
    q, k, v, _, cu = upload(inp)
    kw = dict(cu_seqlens_q=cu, max_seqlen_q=inp.max_seqlen() if inp.varlen else None, tuning=tuning)
    o16, lse16 = FA.fwd(q, k, v, inp.scale, inp.causal, **kw)
    o32 = torch.empty(q.shape, dtype=torch.float32, device=q.device)
    _, lse32 = FA.fwd(q, k, v, inp.scale, inp.causal, out=o32, **kw)
    torch.cuda.synchronize()
    assert torch.equal(o32.to(torch.bfloat16).view(torch.int16), o16.view(torch.int16))
    assert torch.equal(lse32, lse16)
    pairs = [(0, 0), (inp.batch - 1, inp.num_heads - 1)]
    check_heads(inp, o32, lse32, pairs, tag=f"fp32 O {case}", strict=True)


def test_forward_is_bitwise_repeatable():
    inp = I.random_inputs(31, 2, 2048, 4, 128, True, q_std=3.0)
    q, k, v, _, _ = upload(inp)
    outs = [FA.fwd(q, k, v, inp.scale, True) for _ in range(3)]
    torch.cuda.synchronize()
    for o, lse in outs[1:]:
        assert torch.equal(o.view(torch.int16), outs[0][0].view(torch.int16))
        assert torch.equal(lse, outs[0][1])


def test_rescale_threshold_zero_and_eight_agree():
    inp = I.random_inputs(41, 1, 1536, 4, 128, True, q_std=3.0)
    q, k, v, _, _ = upload(inp)
    o8, l8 = FA.fwd(q, k, v, inp.scale, True, tuning=FA.Tuning(0, 8, 2))
    o0, l0 = FA.fwd(q, k, v, inp.scale, True, tuning=FA.Tuning(0, 0, 2))
    torch.cuda.synchronize()
    # Both are checked against the oracle elsewhere.  Between themselves they differ
    # by how the unnormalised weights round to bf16 under the two references: each
    # weight carries a relative error of at most 2^-9 either way, which moves the
    # normalised average by at most 2 * 2^-9 * max_j |v_j - o|; then the bf16
    # rounding of the output itself (up to two units in its last place).
    a8, a0 = o8.float(), o0.float()
    vmax = v.float().abs().amax(dim=(1, 3), keepdim=True)        # per (batch, head)
    ulp = torch.exp2(torch.floor(torch.log2(torch.maximum(a8.abs(), a0.abs()).clamp_min(2 ** -126))) - 7)
    bound = 2 * ulp + 2.0 ** -8 * (vmax + a0.abs())
    excess = ((a8 - a0).abs() - bound).max().item()
    d = (a8 - a0).abs().max().item()
    dl = (l8 - l0).abs().max().item()
    say(f"[lazy vs eager] O max diff {d:.3e} (max excess over the rounding bound {excess:.3e})  "
        f"LSE max diff {dl:.3e}")
    assert excess <= 0.0 and dl <= TOL_LSE
