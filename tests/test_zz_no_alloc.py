"""fa_bwd_noalloc (the backward on the library's static workspace) against fa_bwd on
the same inputs: two calls in a row, the second on a smaller problem, in both dQ
modes.  Deterministic mode must agree bit for bit (same kernels, same order); atomic
mode within the parity bar (its dQ summation order varies between runs)."""
import numpy as np
import pytest
import torch

from tiled_exact_attention_bf16_amd import inputs as I
from tests.gpu_util import TOL_MAX, TOL_MEAN, errors, oracle_forward_tensors, say, upload

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from tiled_exact_attention_bf16_amd import attention as FA


def run_pair(inp, deterministic, grad_dtype):
    q, k, v, do, cu = upload(inp)
    o, lse = oracle_forward_tensors(inp)
    kw = dict(cu_seqlens_q=cu, max_seqlen_q=inp.max_seqlen()) if inp.varlen else {}
    ref = FA.bwd(do, q, k, v, o, lse, inp.scale, inp.causal, deterministic=deterministic, grad_dtype=grad_dtype,
                 **kw)
    got = tuple(torch.full(t.shape, float("nan"), dtype=grad_dtype, device="cuda") for t in (q, k, v))
    FA.bwd_noalloc(do, q, k, v, o, lse, *got, inp.scale, inp.causal, deterministic=deterministic, **kw)
    torch.cuda.synchronize()
    return ref, got


@pytest.mark.parametrize("deterministic", [True, False])
def test_noalloc_backward_matches_fa_bwd_twice(deterministic):
    cases = [I.random_inputs(71, 2, 1000, 4, 128, True, with_do=True),            # larger first
             I.random_varlen_inputs(72, [300, 1, 129, 0, 64], heads=2, head_dim=64, causal=True, with_do=True)]
    for n, inp in enumerate(cases):
        say(f"case noalloc call {n} det={deterministic} {inp.q.shape}")
        for grad_dtype in (torch.float32, torch.bfloat16):
            ref, got = run_pair(inp, deterministic, grad_dtype)
            for name, a, b in zip(("dq", "dk", "dv"), ref, got):
                assert bool(torch.isfinite(b).all()), (n, name)
                if deterministic:
                    assert torch.equal(a.view(torch.int16 if grad_dtype == torch.bfloat16 else torch.int32),
                                       b.view(torch.int16 if grad_dtype == torch.bfloat16 else torch.int32)), (n, name)
                else:
                    mx, mean = errors(b.float().cpu().numpy(), a.float().cpu().numpy().astype(np.float64))
                    assert mx <= TOL_MAX and mean <= TOL_MEAN, (n, name, mx, mean)
    say(f"[noalloc det={deterministic}] two calls in a row agree with fa_bwd")
