"""Fit of the cubic behind the library's polynomial exp2 (the software-exp2
split of the prefill, ``exp2_poly`` in csrc/prefill.hip).

2^x = 2^n * 2^f with n = floor(x) and f = x - n in [0, 1).  The kernel
evaluates 2^f with a polynomial c(f) whose coefficients minimise the largest
relative error max |c(f) / 2^f - 1| over [0, 1].  The fit is the Remez
exchange algorithm for a weighted (relative) error:

* start from Chebyshev-spaced reference points;
* solve the linear system c(x_i) / 2^x_i - 1 = (-1)^i E for c and E;
* move the reference to the alternating extrema of the error on a fine grid;
* repeat until the extrema equioscillate.

``python -m flashattention_forward_amd.exp2_poly_fit`` prints the fp32
coefficients (constant term first) and the error bound.  The library's
constants are these values rounded to fp32.
"""
from __future__ import annotations

import numpy as np

DEGREE = 3


def fit(degree: int = DEGREE, iters: int = 40, grid: int = 200001):
    """(coefficients fp64, constant term first; max relative error on [0, 1])."""
    n = degree + 2
    ref = 0.5 - 0.5 * np.cos(np.pi * np.arange(n) / (n - 1))
    g = np.linspace(0.0, 1.0, grid)
    c = None
    for _ in range(iters):
        a = np.zeros((n, n))
        for i, xi in enumerate(ref):
            a[i, :degree + 1] = xi ** np.arange(degree + 1) / 2.0 ** xi
            a[i, degree + 1] = (-1.0) ** i
        c = np.linalg.solve(a, np.ones(n))[:degree + 1]
        err = np.polyval(c[::-1], g) / 2.0 ** g - 1.0
        # local extrema of the error (and the two end points), merged so that signs alternate
        d = np.diff(err)
        idx = [0] + [i for i in range(1, grid - 1) if d[i - 1] * d[i] <= 0] + [grid - 1]
        sel = []
        for i in idx:
            if sel and np.sign(err[i]) == np.sign(err[sel[-1]]):
                if abs(err[i]) > abs(err[sel[-1]]):
                    sel[-1] = i
            else:
                sel.append(i)
        while len(sel) > n:
            sel.pop(0 if abs(err[sel[0]]) < abs(err[sel[-1]]) else -1)
        if len(sel) == n:
            ref = g[sel]
    err = np.polyval(c[::-1], g) / 2.0 ** g - 1.0
    return c, float(np.abs(err).max())


def coefficients_f32(degree: int = DEGREE) -> np.ndarray:
    """The fitted coefficients rounded to fp32, constant term first."""
    return fit(degree)[0].astype(np.float32)


if __name__ == "__main__":
    c, e = fit()
    print("coefficients (fp32, constant first):", [repr(float(v)) for v in c.astype(np.float32)])
    print("max relative error on [0, 1]: %.3e" % e)
