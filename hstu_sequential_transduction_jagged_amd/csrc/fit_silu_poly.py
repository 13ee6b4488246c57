#!/usr/bin/env python3
"""Fit of the odd polynomial used by the bf16 attention kernel for SiLU on a bounded range.

With y = -log2(e) x, SiLU(x) = -(ln 2 / 2) w(y), w(y) = 2 y s(y), s(y) = 1 / (1 + 2^y).
s(y) - 1/2 is odd, so s(y) = 1/2 - y Q(y^2) and w(y) = y - y^2 P(y^2) with P = 2 Q.
This script fits P of degree 2 in u = y^2 on |y| <= R, minimising the largest relative
error of s (Lawson's iteratively reweighted least squares, which converges to the
minimax fit), and prints the coefficients and the error bound.

    python fit_silu_poly.py [R]
"""
import sys

import numpy as np


def fit(R=2.0, deg=2, iters=200, n=4001):
    y = np.linspace(R / n, R, n)
    s = 1.0 / (1.0 + np.exp2(y))
    u = y * y
    A = np.stack([u ** k for k in range(deg + 1)], axis=1)
    # relative error of s: (y P(u) / 2 - (1/2 - s)) / s, linear in the coefficients of P
    M = (y / 2.0)[:, None] * A / s[:, None]
    t = (0.5 - s) / s
    wgt = np.full(n, 1.0 / n)
    for _ in range(iters):
        sw = np.sqrt(wgt)
        c, *_ = np.linalg.lstsq(M * sw[:, None], t * sw, rcond=None)
        e = np.abs(M @ c - t)
        wgt = wgt * e
        wgt /= wgt.sum()
    return c, float(np.max(np.abs(M @ c - t)))


if __name__ == "__main__":
    R = float(sys.argv[1]) if len(sys.argv) > 1 else 2.0
    c, err = fit(R)
    print("range %.3g  P = [%s]  max relative error of 1/(1+2^y): %.3g"
          % (R, ", ".join("%.10f" % x for x in c), err))
