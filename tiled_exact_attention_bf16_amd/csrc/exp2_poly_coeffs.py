"""Derives the cubic used by the kernels' FMA-only exp2 (constants kExp2P1..P3).

2^f on [0, 1] is approximated by p(f) = 1 + c1 f + c2 f^2 + c3 f^3 (p(0) = 1 keeps
exact powers of two exact).  The coefficients minimise the squared relative error
sum_i ((p(f_i) - 2^f_i) / 2^f_i)^2 over 4,097 Chebyshev nodes of [0, 1], then are
rounded to float32.  Run:  python exp2_poly_coeffs.py
"""
import numpy as np


def coefficients(n: int = 4097):
    i = np.arange(n)
    f = 0.5 - 0.5 * np.cos(np.pi * (i + 0.5) / n)       # Chebyshev nodes on [0, 1]
    w = np.exp2(f)
    a = np.stack([f, f ** 2, f ** 3], axis=1) / w[:, None]
    rhs = 1.0 - 1.0 / w
    c, *_ = np.linalg.lstsq(a, rhs, rcond=None)
    return [float(np.float32(x)) for x in c]


if __name__ == "__main__":
    c = coefficients()
    f = np.linspace(0, 1, 200001)
    p = 1 + f * (c[0] + f * (c[1] + f * c[2]))
    print("c1 = %.9g\nc2 = %.9g\nc3 = %.9g" % tuple(c))
    print("max relative error %.3g" % np.max(np.abs(p / np.exp2(f) - 1)))
