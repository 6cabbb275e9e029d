"""Check build against the library: libfa_gfx950_serial.so waits for every batch of
buffer->LDS loads as soon as it is issued, so no load overlaps any computation.  Its
outputs must equal the library's bit for bit; a difference means some computation read
LDS that a load in flight was still filling (or a buffer was refilled while in use)."""
import contextlib

import numpy as np
import pytest
import torch

from tiled_exact_attention_bf16_amd import _lib as L
from tiled_exact_attention_bf16_amd import inputs as I
from tests.gpu_util import say, upload

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from tiled_exact_attention_bf16_amd import attention as FA


@contextlib.contextmanager
def serial_library():
    """Route the binding's calls through the check build for the duration."""
    normal = L.lib()
    L._lib = L.load(L.SERIAL_LIB_PATH)
    try:
        yield
    finally:
        L._lib = normal


def run(inp, tuning=None):
    q, k, v, do, cu = upload(inp)
    ms = inp.max_seqlen() if inp.varlen else None
    o, lse = FA.fwd(q, k, v, inp.scale, inp.causal, cu_seqlens_q=cu, max_seqlen_q=ms, tuning=tuning)
    dq, dk, dv = FA.bwd(do, q, k, v, o, lse, inp.scale, inp.causal, deterministic=True,
                        cu_seqlens_q=cu, max_seqlen_q=ms)
    torch.cuda.synchronize()
    return [t.view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32).cpu().numpy()
            for t in (o, lse, dq, dk, dv)]


CASES = [
    ("causal B2 S1000 H3 d128", lambda: I.random_inputs(31, 2, 1000, 3, 128, causal=True, with_do=True), None),
    ("full B1 S777 H2 d64", lambda: I.random_inputs(32, 1, 777, 2, 64, causal=False, with_do=True), None),
    ("varlen causal d128", lambda: I.random_varlen_inputs(33, [5, 300, 1100, 64], 2, 128, causal=True,
                                                          with_do=True), None),
    ("causal Lq 40 Lk 3000, key split", lambda: I.random_inputs(34, 2, 40, 2, 128, causal=True, with_do=True,
                                                                seqlen_k=3000), "split"),
    ("causal S600 one query tile per workgroup", lambda: I.random_inputs(35, 1, 600, 2, 128, causal=True,
                                                                         with_do=True), "qt1"),
]


@pytest.mark.parametrize("name,make,variant", CASES, ids=[c[0] for c in CASES])
def test_serial_loads_build_is_bitwise_identical(name, make, variant):
    say(f"case serial-loads {name}")
    inp = make()
    tuning = None
    if variant == "split":
        tuning = FA.Tuning(key_splits=4)
    elif variant == "qt1":
        tuning = FA.Tuning(q_tiles_per_workgroup=1)
    ref = run(inp, tuning)
    with serial_library():
        got = run(inp, tuning)
    for label, a, b in zip(("o", "lse", "dq", "dk", "dv"), ref, got):
        assert np.array_equal(a, b), (name, label, int(np.sum(a != b)))
