"""Pins of the complementary-error-function fit that the GELU epilogue of the linear layers uses
(no GPU): the coefficients in the kernel source are the ones the fit script produces, the fit
meets its stated error bound against scipy's erfc, and the GELU built from it matches the exact
erf form in float64 to that bound."""

import importlib.util
import math
import os
import re

import numpy as np
from scipy.special import erf, erfc

ROOT = os.path.join(os.path.dirname(__file__), "..", "vision_transformer_windowed_window_amd", "csrc")


def _fit_module():
    spec = importlib.util.spec_from_file_location("fit_erfc", os.path.join(ROOT, "fit_erfc.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _kernel_coefficients():
    src = open(os.path.join(ROOT, "wattn_model.hip")).read()
    body = src[src.index("float gelu_erf(float x)"):]
    body = body[:body.index("\n}\n")]
    first = float(re.search(r"float p = ([-+0-9.e]+)f;", body).group(1))
    rest = [float(v) for v in re.findall(r"p = fmaf\(p, t, ([-+0-9.e]+)f\);", body)]
    return np.array(([first] + rest)[::-1])  # c0 .. c7


def test_kernel_coefficients_are_the_fit():
    c = _fit_module().fit()
    k = _kernel_coefficients()
    assert k.shape == c.shape
    np.testing.assert_allclose(k, c, rtol=1e-8, atol=1e-9)


def test_fit_error_bound():
    rel64, rel32 = _fit_module().check(_kernel_coefficients())
    assert rel64 < 6.5e-7 and rel32 < 3e-5


def test_gelu_from_the_fit_matches_the_erf_form():
    c = _kernel_coefficients()
    x = np.linspace(-12.0, 12.0, 200001)
    z = np.abs(x) / math.sqrt(2.0)
    t = 1.0 / (1.0 + z / 2.0)
    q = t * np.exp(-z * z + np.polynomial.polynomial.polyval(t, c))
    got = 0.5 * x * np.where(x >= 0, 2.0 - q, q)
    ref = 0.5 * x * (1.0 + erf(x / math.sqrt(2.0)))
    # relative to |x|: the GELU error is 0.5 |x| times the erfc error, and erfc <= 2
    assert np.max(np.abs(got - ref) / np.maximum(np.abs(x), 1e-30)) < 1e-6
    # relative to the value for negative x, where GELU is small: erfc's relative error carries
    # over (the reference written as 0.5 x erfc(|x| / sqrt 2), which has no cancellation there)
    neg = x < -1e-3
    ref_neg = 0.5 * x[neg] * erfc(z[neg])
    assert np.max(np.abs(got[neg] / ref_neg - 1.0)) < 1e-6
    assert np.all(np.abs(erfc(z) - q) <= 6.5e-7 * erfc(z) + 1e-300)
