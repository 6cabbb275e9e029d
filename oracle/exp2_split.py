"""Model of the FMA-only exp2 split (fp32), with its own polynomial fit.

TEST INFRASTRUCTURE (only tests/, ``__graft_entry__.smoke()`` and bench.py's
``cpu_baseline`` leg may use oracle/).  Shares no code or constants with the HIP
kernels, which carry their own independently fitted coefficients.

The method (fdeinterviews.com FA4 summary, "Software exponentials" bullet;
lecompute.fr FA4 article, section "Move some exponential work to different
units"): 2**x is formed with multiplies and adds only -- x is split into its
integer part and its fractional part, a cubic in the fraction approximates 2**f,
and the integer is added into the float's exponent bits.  The pages state the
accuracy this reaches against the hardware unit once both are rounded to bf16: a
difference of at most one bf16 ulp for all but about 1% of arguments.

Readings where the pages leave a step open:
  * the split is floor-based: j = floor(x), f = x - j in [0, 1];
  * the cubic is this module's own minimax fit of 2**f on [0, 1] in relative
    error, with p(0) = 1 exactly (so integer x give exact powers of two);
  * the float is IEEE binary32; results below 2**-126 (x < -126) flush to 0, as
    do x = -inf (masked scores);
  * the arithmetic is fp32 with a separate rounding after every multiply and add
    (a fused multiply-add would only round less).
"""
from __future__ import annotations

import functools

import numpy as np


@functools.lru_cache(maxsize=None)
def fit_cubic(n_grid: int = 4097) -> tuple:
    """Minimax (relative error) cubic for 2**f on [0,1] with p(0) = 1.

    Solved as a linear program over (c1, c2, c3, t): minimise t subject to
    |p(f_i) / 2**f_i - 1| <= t on a dense grid.  Returns (c0, c1, c2, c3) as
    float32-representable Python floats, and caches the result.
    """
    from scipy.optimize import linprog

    f = np.linspace(0.0, 1.0, n_grid)
    w = np.exp2(f)
    # p(f) = 1 + c1 f + c2 f^2 + c3 f^3 ;  (p - w)/w <= t  and  (w - p)/w <= t
    a = np.stack([f / w, f ** 2 / w, f ** 3 / w], axis=1)
    r = 1.0 - 1.0 / w                         # (1 - w)/w moved to the right-hand side
    a_ub = np.concatenate([np.concatenate([a, -np.ones((n_grid, 1))], axis=1),
                           np.concatenate([-a, -np.ones((n_grid, 1))], axis=1)])
    b_ub = np.concatenate([r, -r])
    res = linprog(c=[0, 0, 0, 1], A_ub=a_ub, b_ub=b_ub, bounds=[(None, None)] * 4, method="highs")
    if not res.success:
        raise RuntimeError("exp2 cubic fit failed: " + res.message)
    c1, c2, c3, _ = res.x
    return tuple(float(np.float32(c)) for c in (1.0, c1, c2, c3))


def exp2_split(x: np.ndarray, coeffs=None) -> np.ndarray:
    """2**x for float32 x by integer/fraction split and a cubic on the fraction."""
    if coeffs is None:
        coeffs = fit_cubic()
    c0, c1, c2, c3 = (np.float32(c) for c in coeffs)
    x = np.asarray(x, dtype=np.float32)
    with np.errstate(invalid="ignore", over="ignore"):
        xc = np.where(x < np.float32(-126.0), np.float32(-126.0), x).astype(np.float32)
        j = np.floor(xc).astype(np.float32)
        f = (xc - j).astype(np.float32)
        p = c3
        p = (p * f).astype(np.float32) + c2
        p = (p * f).astype(np.float32) + c1
        p = (p * f).astype(np.float32) + c0
        p = np.asarray(p, dtype=np.float32)
        bits = p.view(np.int32) + (j.astype(np.int32) << 23)
    out = bits.view(np.float32)
    return np.where(x < np.float32(-126.0), np.float32(0.0), out).astype(np.float32)


def bf16_ulp_distance(a32: np.ndarray, b32: np.ndarray) -> np.ndarray:
    """|difference| in bf16 units in the last place after RNE-rounding both to bf16.

    Both inputs must be non-negative finite float32 (as exponentials are).
    """
    def rne(x):
        u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.int64)
        return (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return np.abs(rne(a32) - rne(b32))
