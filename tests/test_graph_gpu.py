"""HIP graph capture of the forward and the allocation-free backward (the callers
fa_bwd_noalloc is for): every replay must reproduce the eager results bit for bit
(deterministic dQ), with eager work and synchronisations between the replays."""
import pytest
import torch

from tiled_exact_attention_bf16_amd import inputs as I
from tests.gpu_util import say, upload

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from tiled_exact_attention_bf16_amd import attention as FA


def bits(t: torch.Tensor) -> torch.Tensor:
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def test_graph_replays_match_eager():
    say("case graph capture of fwd + bwd_noalloc, causal B1 S700 H2 d128")
    inp = I.random_inputs(41, 1, 700, 2, 128, causal=True, with_do=True)
    q, k, v, do, _ = upload(inp)
    s = inp.scale
    ws = FA.fwd_workspace(q, k, v, s, True)
    o = torch.empty_like(q)
    lse = torch.empty((1, 2, 700), dtype=torch.float32, device="cuda")
    dq, dk, dv = (torch.empty(t.shape, dtype=torch.float32, device="cuda") for t in (q, k, v))

    def body():
        FA.fwd(q, k, v, s, True, out=o, lse=lse, workspace=ws)
        FA.bwd_noalloc(do, q, k, v, o, lse, dq, dk, dv, s, True, deterministic=True)

    # eager reference (it also runs the library's once-per-device set-up outside the capture)
    body()
    torch.cuda.synchronize()
    ref = [bits(t).clone() for t in (o, lse, dq, dk, dv)]
    # warm up on a side stream, then capture
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        body()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        body()
    torch.cuda.synchronize()
    # replays, each after the outputs were poisoned and other eager work ran
    other = I.random_inputs(42, 1, 300, 2, 128, causal=False)
    q2, k2, v2, _, _ = upload(other)
    for rep in range(3):
        for t in (o, lse, dq, dk, dv):
            t.fill_(float("nan"))
        FA.fwd(q2, k2, v2, other.scale, False)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, r, t in zip(("o", "lse", "dq", "dk", "dv"), ref, (o, lse, dq, dk, dv)):
            assert torch.equal(r, bits(t)), (rep, name)
