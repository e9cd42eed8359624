"""Coefficients of the complementary error function used by the GELU epilogue of the linear
layers (wattn_model.hip, gelu_erf).

Form: erfc(z) = t * exp(-z^2 + P(t)) with t = 1 / (1 + z / 2), z >= 0, and P a polynomial of
degree 7 in t.  P is fitted here to ln(erfc(z) / t) + z^2 on z in [0, 10] (t in [1/6, 1]) by
iteratively reweighted least squares (Lawson's algorithm), which drives the fit towards the
minimax error in the exponent; that error is the relative error of erfc.  Run with
`python fit_erfc.py`; it prints the coefficients c0 .. c7 and the largest relative error of
erfc over z in [0, 9.5], in float64 and in a float32 evaluation of the kernel's formula.
"""

import numpy as np
from scipy.special import erfc

DEG = 7
ZMAX = 10.0


def fit(deg=DEG, zmax=ZMAX, n=20000, iters=200):
    lo = 1.0 / (1.0 + zmax / 2.0)
    t = lo + (1.0 - lo) * (0.5 + 0.5 * np.cos(np.linspace(0.0, np.pi, n)))
    z = 2.0 * (1.0 / t - 1.0)
    f = np.log(erfc(z) / t) + z * z
    V = np.vander(t, deg + 1, increasing=True)
    w = np.ones_like(t)
    for _ in range(iters):
        sw = np.sqrt(w)
        c, *_ = np.linalg.lstsq(V * sw[:, None], f * sw, rcond=None)
        w = w * np.abs(V @ c - f)
        w /= w.sum()
    return c


def check(c):
    z = np.linspace(0.0, 9.5, 400001)
    t = 1.0 / (1.0 + z / 2.0)
    q = t * np.exp(-z * z + np.polynomial.polynomial.polyval(t, c))
    rel64 = np.abs(q / erfc(z) - 1.0).max()
    z32 = z.astype(np.float32)
    t32 = np.float32(1.0) / (np.float32(1.0) + np.float32(0.5) * z32)
    p = np.float32(c[-1])
    for a in c[-2::-1]:  # Horner with fused multiply-adds (one rounding each)
        p = (p.astype(np.float64) * t32.astype(np.float64) + np.float64(np.float32(a))).astype(np.float32)
    arg = (p.astype(np.float64) - (z32 * z32).astype(np.float64)).astype(np.float32)
    q32 = t32 * np.exp(arg.astype(np.float64)).astype(np.float32)
    rel32 = np.abs(q32.astype(np.float64) / erfc(z32.astype(np.float64)) - 1.0).max()
    return rel64, rel32


if __name__ == "__main__":
    c = fit()
    rel64, rel32 = check(c)
    for i, a in enumerate(c):
        print("c%d = %.9ef" % (i, a))
    print("max relative error of erfc on [0, 9.5]: %.2e (float64), %.2e (float32)" % (rel64, rel32))
