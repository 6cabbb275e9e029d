"""Device probe of the forward's two exponentials (fa_exp2_probe) on every fp32 input of
[-126, 8] (2.21e9 bit patterns) and a 2^24-point uniform grid.

The software 2^x (split into integer and fraction, cubic on the fraction, integer
added to the exponent bits; FA4 summary page, "Software exponentials" bullet) and the
hardware v_exp_f32, as the forward kernel evaluates them, each within one bf16 ulp of
the library exp2 (fp64) on at least the share of inputs the pages give; the software
path also against the hardware unit, which is what the pages compare it with.
"""
import json
import os

import numpy as np
import pytest
import torch

from tests.gpu_util import say

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from tiled_exact_attention_bf16_amd import attention as FA

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_figures.json")))["software_exp2"]


def _bf16_bits_t(x32: "torch.Tensor") -> "torch.Tensor":
    """Round-to-nearest-even bf16 bit patterns of non-negative float32 values (int64)."""
    u = x32.contiguous().view(torch.int32).to(torch.int64) & 0xFFFFFFFF
    return (u + 0x7FFF + ((u >> 16) & 1)) >> 16


def _chunks(name: str, chunk: int = 1 << 27):
    """Every fp32 bit pattern of the range, in chunks (device tensors), or the grid."""
    if name == "uniform grid":  # 2^24 points uniform in value over [-126, 8]
        yield torch.linspace(-126.0, 8.0, 1 << 24, dtype=torch.float64, device="cuda").to(torch.float32)
        return
    if name == "negative":      # every pattern of [-126, 0): 0x80000001 .. 0xC2FC0000 (and -0)
        lo, hi = 0x80000000, int(np.array(-126.0, dtype=np.float32).view(np.uint32))
    else:                       # every pattern of [0, 8]: 0x00000000 .. 0x41000000
        lo, hi = 0, int(np.array(8.0, dtype=np.float32).view(np.uint32))
    for a in range(lo, hi + 1, chunk):
        b = min(hi + 1, a + chunk)
        bits = torch.arange(a, b, dtype=torch.int64, device="cuda")
        bits = torch.where(bits >= 1 << 31, bits - (1 << 32), bits).to(torch.int32)
        yield bits.view(torch.float32)


@pytest.mark.parametrize("name", ["negative", "non-negative", "uniform grid"])
def test_exp2_probe_dense_sweep(name):
    # every fp32 bit pattern of [-126, 8] (2.21e9 inputs over the two ranges) plus a
    # 2^24-point uniform grid; reference: fp64 exp2 rounded to fp32, then to bf16
    n = ok_poly = ex_poly = ok_hw = ex_hw = ok_pair = ex_pair = 0
    worst = 0
    for x in _chunks(name):
        y_poly, y_hw = FA.exp2_probe(x)
        ref = torch.exp2(x.to(torch.float64)).to(torch.float32)
        bp, bh, br = _bf16_bits_t(y_poly), _bf16_bits_t(y_hw), _bf16_bits_t(ref)
        assert bool(torch.isfinite(y_poly).all()) and bool((y_poly > 0).all())
        d_poly, d_hw, d_pair = (bp - br).abs(), (bh - br).abs(), (bp - bh).abs()
        n += x.numel()
        ok_poly += int((d_poly <= 1).sum()); ex_poly += int((d_poly == 0).sum())
        ok_hw += int((d_hw <= 1).sum()); ex_hw += int((d_hw == 0).sum())
        ok_pair += int((d_pair <= 1).sum()); ex_pair += int((d_pair == 0).sum())
        worst = max(worst, int(d_poly.max()))
        del x, y_poly, y_hw, ref, bp, bh, br, d_poly, d_hw, d_pair
    say(f"[exp2 {name}] {n} inputs | software: <=1 ulp {ok_poly / n:.6f}, exact {ex_poly / n:.6f}, max {worst} | "
        f"v_exp_f32: <=1 ulp {ok_hw / n:.6f}, exact {ex_hw / n:.6f} | "
        f"software vs v_exp_f32: <=1 ulp {ok_pair / n:.6f}, exact {ex_pair / n:.6f}")
    share = GOLDEN["fraction_of_inputs"]
    assert ok_poly / n >= share and ok_hw / n >= share and ok_pair / n >= share
    if name != "uniform grid":
        expected = {"negative": 0xC2FC0000 - 0x80000000 + 1, "non-negative": 0x41000000 + 1}[name]
        assert n == expected


def _probe(xs: np.ndarray):
    x = torch.from_numpy(np.ascontiguousarray(xs, dtype=np.float32)).cuda()
    y_poly, y_hw = FA.exp2_probe(x)
    torch.cuda.synchronize()
    return y_poly.cpu().numpy(), y_hw.cpu().numpy()


def test_exp2_probe_special_values():
    ints = np.arange(-126, 9, dtype=np.float32)
    xs = np.concatenate([ints, np.array([-np.inf, -127.5, -1000.0], dtype=np.float32)])
    y_poly, y_hw = _probe(xs)
    n = len(ints)
    exact = np.exp2(ints.astype(np.float64)).astype(np.float32)
    # the cubic has p(0) = 1, so every power of two is exact, and a weight at the
    # running maximum (x = 0) is exactly 1 on either path
    assert np.array_equal(y_poly[:n], exact)
    zero = int(np.flatnonzero(ints == 0)[0])
    assert y_poly[zero] == 1.0 and y_hw[zero] == 1.0
    # masked scores (-inf) and arguments below the normal range give weight 0
    assert y_poly[n:].tolist() == [0.0, 0.0, 0.0]
    assert y_hw[n] == 0.0 and y_hw[n + 2] == 0.0
    say(f"[exp2 integers] v_exp_f32 exact on {np.mean(y_hw[:n] == exact):.3f} of 2^-126..2^8")
