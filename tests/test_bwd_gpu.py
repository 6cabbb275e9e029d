"""Backward parity (atomic and deterministic dQ) against the fp64 oracle, and the
deterministic mode's bitwise reproducibility."""
import numpy as np
import pytest
import torch

from tiled_exact_attention_bf16_amd import inputs as I
from tests.gpu_util import (TOL_MAX, TOL_MEAN, bf16_rounding_floor, bf16_rounding_max, errors, gpu_head,
                            named_inputs, oracle_bwd_head, oracle_forward_tensors, oracle_map, say, upload)

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from tiled_exact_attention_bf16_amd import attention as FA


def run_bwd_on_oracle_forward(inp, deterministic, grad_dtype=torch.float32, cu_k=None):
    """The backward alone: O (bf16) and LSE (fp32) come from the oracle's forward."""
    q, k, v, do, cu = upload(inp)
    o, lse = oracle_forward_tensors(inp)
    kw = {}
    if inp.varlen:
        kw = dict(cu_seqlens_q=cu, max_seqlen_q=inp.max_seqlen())
        if cu_k is not None:
            kw.update(cu_seqlens_k=cu_k, max_seqlen_k=inp.max_seqlen_k())
    dq, dk, dv = FA.bwd(do, q, k, v, o, lse, inp.scale, inp.causal, deterministic=deterministic,
                        grad_dtype=grad_dtype, **kw)
    torch.cuda.synchronize()
    return dq, dk, dv


def run_fwd_bwd(inp, deterministic, grad_dtype=torch.float32):
    q, k, v, do, cu = upload(inp)
    ms = inp.max_seqlen() if inp.varlen else None
    o, lse = FA.fwd(q, k, v, inp.scale, inp.causal, cu_seqlens_q=cu, max_seqlen_q=ms)
    dq, dk, dv = FA.bwd(do, q, k, v, o, lse, inp.scale, inp.causal, deterministic=deterministic,
                        grad_dtype=grad_dtype, cu_seqlens_q=cu, max_seqlen_q=ms)
    torch.cuda.synchronize()
    return dq, dk, dv


def check_grads(inp, grads, pairs, tag, strict=False, cache_key=None):
    """strict (the named workloads, run end to end from the GPU forward): the exact fp64
    oracle at the literal bar.

    Otherwise (edge-case shapes: a handful of keys per row, so large weights and large
    gradients; run by run_bwd_on_oracle_forward): the oracle whose row terms
    D_i = dO_i . O_i use the oracle's own O rounded to bf16 -- the O that backward was
    handed -- again at the literal bar.  bf16 gradient outputs also carry their own
    rounding (no bf16 output can beat bf16 of the oracle), which is added to the bar."""
    worst = {}
    refs = oracle_map(lambda bh: oracle_bwd_head(inp, bh[0], bh[1], o_bf16=not strict, cache_key=cache_key), pairs)
    for (b, h), ref in zip(pairs, refs):
        for name, g, r in zip(("dq", "dk", "dv"), grads, ref):
            got = gpu_head(g, inp, b, h, "q" if name == "dq" else "k")
            assert np.all(np.isfinite(got)), (tag, name, b, h)
            mx, mean = errors(got, r)
            w = worst.get(name, (0.0, 0.0))
            worst[name] = (max(w[0], mx), max(w[1], mean))
            relax = g.dtype == torch.bfloat16 and not strict
            floor_max = bf16_rounding_max(r) if relax else 0.0
            floor_mean = bf16_rounding_floor(r) if relax else 0.0
            assert mx <= TOL_MAX + floor_max and mean <= TOL_MEAN + floor_mean, (tag, name, b, h, mx, mean)
    say(f"[bwd {tag}] " + "  ".join(f"{k} {v[0]:.3e}/{v[1]:.3e}" for k, v in worst.items()))


@pytest.mark.parametrize("deterministic", [False, True])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("s", [1, 17, 128, 129, 300, 1000])
def test_small_shapes(s, causal, d, deterministic):
    inp = I.random_inputs(200 + s, 2, s, 2, d, causal, with_do=True)
    say(f"case s={s} causal={causal} d={d} det={deterministic}")
    grads = run_bwd_on_oracle_forward(inp, deterministic)
    check_grads(inp, grads, [(b, h) for b in range(2) for h in range(2)], f"s{s}c{int(causal)}d{d}det{int(deterministic)}")


@pytest.mark.parametrize("deterministic", [False, True])
@pytest.mark.parametrize("lq,lk", [(7, 300), (300, 129), (64, 1000), (1000, 64), (1, 257), (130, 200)])
def test_causal_unequal_lengths(lq, lk, deterministic):
    # bottom-right causal alignment; with lq > lk the first lq - lk rows see no key
    inp = I.random_inputs(400 + lq + lk, 2, lq, 2, 128, True, with_do=True, seqlen_k=lk)
    say(f"case causal lq={lq} lk={lk} det={deterministic}")
    grads = run_bwd_on_oracle_forward(inp, deterministic)
    check_grads(inp, grads, [(b, h) for b in range(2) for h in range(2)], f"causal{lq}x{lk}det{int(deterministic)}")


@pytest.mark.parametrize("deterministic", [False, True])
@pytest.mark.parametrize("causal", [False, True])
def test_varlen_separate_key_lengths(causal, deterministic):
    q_lens = [1, 0, 5, 64, 130, 1, 17, 300]
    k_lens = [300, 7, 410, 64, 200, 0, 900, 129]
    inp = I.random_varlen_qk_inputs(78, q_lens, k_lens, heads=2, head_dim=128, causal=causal)
    rng = np.random.default_rng(79)
    inp.do = I.f32_to_bf16_bits(rng.standard_normal(inp.q.shape, dtype=np.float32))
    say(f"case varlen q/k lengths causal={causal} det={deterministic}")
    grads = run_bwd_on_oracle_forward(inp, deterministic, cu_k=torch.from_numpy(inp.cu_seqlens_k).cuda())
    check_grads(inp, grads, [(b, h) for b in range(len(q_lens)) for h in range(2)],
                f"varlenqk c{int(causal)}det{int(deterministic)}")


@pytest.mark.parametrize("deterministic", [False, True])
def test_varlen_ragged(deterministic):
    lens = [0, 1, 5, 128, 129, 300, 17, 0, 256, 511]
    inp = I.random_varlen_inputs(12, lens, heads=2, head_dim=128, causal=True, with_do=True)
    say(f"case varlen det={deterministic}")
    grads = run_bwd_on_oracle_forward(inp, deterministic)
    check_grads(inp, grads, [(b, h) for b in range(len(lens)) for h in range(2)], f"varlen det{int(deterministic)}")


def test_bf16_gradient_outputs():
    inp = I.random_inputs(300, 1, 512, 2, 128, True, with_do=True)
    grads = run_bwd_on_oracle_forward(inp, False, grad_dtype=torch.bfloat16)
    assert all(g.dtype == torch.bfloat16 for g in grads)
    check_grads(inp, grads, [(0, 0), (0, 1)], "bf16-out")


@pytest.mark.parametrize("deterministic", [False, True])
def test_config_c5_every_head(deterministic):
    # all 32 (batch, head) pairs on every row and key, against the exact oracle at the
    # literal bar; the oracle's gradients are computed once for both dQ modes
    inp = named_inputs("c5")
    say(f"case c5 det={deterministic}: all {inp.batch * inp.num_heads} (batch, head) pairs")
    grads = run_fwd_bwd(inp, deterministic)
    for g in grads:
        assert bool(torch.isfinite(g).all())
    check_grads(inp, grads, [(b, h) for b in range(inp.batch) for h in range(inp.num_heads)],
                f"c5 det{int(deterministic)}", strict=True, cache_key="c5")


@pytest.mark.parametrize("deterministic", [False, True])
@pytest.mark.parametrize("grad_dtype", [torch.float32, torch.bfloat16])
def test_canaries_and_strided_views(deterministic, grad_dtype):
    # inputs and gradients as strided views that skip a guard head, every output buffer
    # followed by a guard region, all poisoned with NaN beforehand, and a NaN-filled
    # workspace (its contents are ignored on entry): the gradients must be finite and
    # correct and no guard element may change
    inp = I.random_inputs(61, 2, 333, 3, 128, True, with_do=True)
    q, k, v, do, _ = upload(inp)
    B, S, H, D = q.shape

    def widened(t):
        big = torch.zeros((B, S, H + 1, D), dtype=t.dtype, device="cuda")
        big[:, :, 1:] = t
        return big[:, :, 1:]

    qv, kv, vv, dov = widened(q), widened(k), widened(v), widened(do)
    assert not qv.is_contiguous()
    o_ref, lse = oracle_forward_tensors(inp)
    o_big = torch.full((B, S, H + 1, D), float("nan"), dtype=torch.bfloat16, device="cuda")
    o = o_big[:, :, 1:]
    o.copy_(o_ref)
    nan = float("nan")
    bigs = [torch.full((B * S * (H + 1) * D + 4096,), nan, dtype=grad_dtype, device="cuda") for _ in range(3)]
    views = [t[: B * S * (H + 1) * D].view(B, S, H + 1, D)[:, :, 1:] for t in bigs]
    ws = torch.full((64 << 20,), 0xFF, dtype=torch.uint8, device="cuda")   # NaN bit patterns
    dq, dk, dv = FA.bwd(dov, qv, kv, vv, o, lse, inp.scale, True, deterministic=deterministic,
                        grad_dtype=grad_dtype, dq=views[0], dk=views[1], dv=views[2], workspace=ws)
    torch.cuda.synchronize()
    for name, big in zip(("dq", "dk", "dv"), bigs):
        body = big[: B * S * (H + 1) * D].view(B, S, H + 1, D)
        assert bool(torch.isnan(body[:, :, 0]).all()), f"{name}: write into the skipped head"
        assert bool(torch.isnan(big[B * S * (H + 1) * D:]).all()), f"{name}: write past the buffer"
    assert bool(torch.isnan(o_big[:, :, 0]).all()), "the backward wrote into O's skipped head"
    check_grads(inp, (dq, dk, dv), [(b, h) for b in range(B) for h in range(H)],
                f"canaries det{int(deterministic)} {str(grad_dtype)[6:]}")


def test_deterministic_mode_is_bitwise_reproducible():
    inp = named_inputs("c5")
    q, k, v, do, _ = upload(inp)
    o, lse = FA.fwd(q, k, v, inp.scale, True)
    first = FA.bwd(do, q, k, v, o, lse, inp.scale, True, deterministic=True)
    first = [g.clone() for g in first]
    for rep in range(5):
        again = FA.bwd(do, q, k, v, o, lse, inp.scale, True, deterministic=True)
        torch.cuda.synchronize()
        for a, b in zip(first, again):
            assert torch.equal(a.view(torch.int32), b.view(torch.int32)), rep
    say("[deterministic] 5 repeats bitwise identical on c5")
