"""Device probe of the forward's two exponentials (fa_exp2_probe) on a dense sweep.

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


def _bf16_bits(x32: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even bf16 bit patterns of non-negative float32 values."""
    u = np.ascontiguousarray(x32, dtype=np.float32).view(np.uint32).astype(np.int64)
    return (u + 0x7FFF + ((u >> 16) & 1)) >> 16


def _ulps(a32: np.ndarray, b32: np.ndarray) -> np.ndarray:
    return np.abs(_bf16_bits(a32) - _bf16_bits(b32))


def _sweep(name: str) -> np.ndarray:
    if name == "negative":   # every 61st fp32 bit pattern of [-126, 0)
        start = int(np.array(-126.0, dtype=np.float32).view(np.uint32))
        return np.arange(start, 0x80000000, -61, dtype=np.int64).astype(np.uint32).view(np.float32)
    if name == "non-negative":  # every 61st fp32 bit pattern of [0, 8]
        return np.arange(0, int(np.float32(8.0).view(np.uint32)) + 1, 61, dtype=np.uint32).view(np.float32)
    return np.linspace(-126.0, 8.0, 1 << 22, dtype=np.float32)  # uniform in value


def _probe(xs: np.ndarray):
    x = torch.from_numpy(np.ascontiguousarray(xs, dtype=np.float32)).cuda()
    y_poly, y_hw = FA.exp2_probe(x)
    torch.cuda.synchronize()
    return y_poly.cpu().numpy(), y_hw.cpu().numpy()


@pytest.mark.parametrize("name", ["negative", "non-negative", "uniform grid"])
def test_exp2_probe_dense_sweep(name):
    xs = _sweep(name)
    say(f"case exp2 sweep {name}: {len(xs)} inputs")
    y_poly, y_hw = _probe(xs)
    ref = np.exp2(xs.astype(np.float64)).astype(np.float32)
    assert np.all(np.isfinite(y_poly)) and np.all(y_poly > 0)
    share = GOLDEN["fraction_of_inputs"]
    d_poly, d_hw, d_pair = _ulps(y_poly, ref), _ulps(y_hw, ref), _ulps(y_poly, y_hw)
    say(f"[exp2 {name}] software: <=1 ulp {np.mean(d_poly <= 1):.6f}, exact {np.mean(d_poly == 0):.6f}, "
        f"max {d_poly.max()} | v_exp_f32: <=1 ulp {np.mean(d_hw <= 1):.6f}, exact {np.mean(d_hw == 0):.6f} | "
        f"software vs v_exp_f32: <=1 ulp {np.mean(d_pair <= 1):.6f}, exact {np.mean(d_pair == 0):.6f}")
    assert np.mean(d_poly <= GOLDEN["max_bf16_ulp"]) >= share
    assert np.mean(d_hw <= GOLDEN["max_bf16_ulp"]) >= share
    assert np.mean(d_pair <= GOLDEN["max_bf16_ulp"]) >= share


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
