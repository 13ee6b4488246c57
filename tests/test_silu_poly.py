"""The bf16 attention kernels replace SiLU by an odd polynomial on tiles where a
Cauchy-Schwarz bound keeps |y| (y = -log2(e) x) inside a fixed range.  These host checks
read the constants from the kernels' shared header and bound the approximation error in fp64
against the exact SiLU; the kernel's parity tests then check the result end to end."""
import os
import re

import numpy as np

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                   "hstu_sequential_transduction_jagged_amd", "csrc", "hstu_internal.h")


def _constants():
    text = open(SRC).read()
    get = lambda name: float(re.search(r"\b%s = (-?[0-9.e+-]+)f" % name, text).group(1))
    return get("kPolyRange"), [get("kP0"), get("kP1"), get("kP2")]


def _w_poly(y, P):
    u = y * y
    return y - u * (P[0] + u * (P[1] + u * P[2]))


def test_polynomial_relative_error_bound():
    R, P = _constants()
    y = np.linspace(-R, R, 200001)
    x = -y / np.log2(np.e)
    silu = x / (1.0 + np.exp(-x))
    approx = -(np.log(2.0) / 2.0) * _w_poly(y, P)
    nz = y != 0
    rel = np.abs(approx[nz] - silu[nz]) / np.abs(silu[nz])
    # far below bf16's unit roundoff 2^-8 = 3.9e-3, which P is rounded to anyway
    assert rel.max() < 1e-4, rel.max()
    assert approx[~nz][0] == 0.0


def test_polynomial_limits():
    R, P = _constants()
    # near 0, s(y) = 1/2 - (ln 2 / 4) y + O(y^3), so P(0) is close to ln(2) / 2 (the minimax
    # fit trades a little accuracy there for the ends of the range)
    assert abs(P[0] - np.log(2.0) / 2.0) < 1e-3
    # the fit is odd in y around the SiLU's symmetric part: w(y) - w(-y) = 2 y exactly
    y = np.linspace(0, R, 101)
    assert np.allclose(_w_poly(y, P) - _w_poly(-y, P), 2 * y, rtol=0, atol=1e-14)


def test_fit_script_reproduces_constants():
    import importlib.util
    spec = importlib.util.spec_from_file_location(
        "fit_silu_poly", os.path.join(os.path.dirname(SRC), "fit_silu_poly.py"))
    m = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(m)
    R, P = _constants()
    c, err = m.fit(R)
    assert np.allclose(c, P, rtol=1e-6, atol=1e-9), (c, P)
    assert err < 1e-4


def _const(name):
    text = open(SRC).read()
    return float(re.search(r"\b%s = (-?[0-9.e+-]+)f" % name, text).group(1))


def test_far_form_relative_error_bound():
    """ALiBi tiles whose bound puts every y at or above kFarExpY use w = 2 y e, e = 2^-y, for the
    exact w = 2 y e / (1 + e): their ratio is 1 + e, a relative error e <= 2^-16."""
    y0 = _const("kFarExpY")
    y = np.linspace(y0, 140.0, 400001)
    e = 2.0 ** -y
    exact = 2.0 * y * e / (1.0 + e)
    rel = np.abs(2.0 * y * e - exact) / exact
    assert y0 >= 16.0 and rel.max() <= 2.0 ** -16 * (1 + 1e-9), rel.max()


def test_far_cut_weight_bound():
    """Pairs with y >= kAlibiFarY are skipped; w decreases for y > 1/ln 2, so each skipped
    weight is at most w(kAlibiFarY) < 7e-18."""
    yc = _const("kAlibiFarY")
    y = np.linspace(yc, 4 * yc, 100001)
    w = 2.0 * y / (1.0 + 2.0 ** y)
    assert np.all(np.diff(w) < 0) and w[0] < 7e-18, w[0]
