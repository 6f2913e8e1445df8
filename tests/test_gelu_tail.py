"""The FFN middle kernels' GELU (csrc/butterfly_impl.hpp, gelu_erf): the exact
erf form h Phi(h) evaluated as relu(h) - |h| Q(|h|) with log2 Q a fitted
degree-7 polynomial.  Its constants must be those the committed fit prints
(csrc/gelu_tail_fit.py), and the formula, evaluated step by step in float32 as
the kernel does (fused multiply-adds rounded once), must stay within the stated
bound of the exact GELU (ButterflyViT pt page §2: GELU between the FFN's two
projections; the bound is far below the bf16 rounding of the kernels' output)."""
import os
import re
import sys

import numpy as np
from scipy.special import ndtr

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "compressed_mixture_experts_amd", "csrc")


def header_constants():
    src = open(os.path.join(CSRC, "butterfly_impl.hpp")).read()
    body = src[src.index("float gelu_erf(float h)"):]
    body = body[:body.index("\n}")]
    clamp = float(re.search(r"fmed3f\(fabsf\(h\), 0\.0f, ([0-9.eE+-]+)f\)", body).group(1))
    lead = float(re.search(r"float p = ([0-9.eE+-]+)f;", body).group(1))
    rest = [float(v) for v in re.findall(r"p = fmaf\(p, a, ([0-9.eE+-]+)f\);", body)]
    return clamp, np.array([lead] + rest, dtype=np.float32)[::-1]   # ascending powers


def kernel_gelu(h, clamp, c):
    h = np.asarray(h, dtype=np.float32)
    a = np.minimum(np.abs(h), np.float32(clamp))
    p = np.full_like(a, c[-1])
    for ci in c[-2::-1]:
        p = (p.astype(np.float64) * a + np.float64(ci)).astype(np.float32)
    q = np.exp2(p.astype(np.float64)).astype(np.float32)
    aq = (a.astype(np.float64) * q).astype(np.float32)
    s = (h.astype(np.float64) + np.abs(h)).astype(np.float32)
    return (0.5 * s.astype(np.float64) - aq).astype(np.float32)


def test_constants_match_the_fit():
    sys.path.insert(0, CSRC)
    try:
        import gelu_tail_fit as fit
    finally:
        sys.path.pop(0)
    clamp, c = header_constants()
    assert clamp == fit.A and len(c) == fit.DEGREE + 1
    np.testing.assert_array_equal(c, fit.fit())


def test_error_bound_against_exact_gelu():
    clamp, c = header_constants()
    h = np.linspace(-12.0, 12.0, 2_400_001).astype(np.float32)
    h64 = h.astype(np.float64)
    exact = h64 * ndtr(h64)
    err = np.abs(kernel_gelu(h, clamp, c) - exact)
    assert np.all(err <= 2e-6 * np.abs(h64) + 1e-7), err.max()
    big = np.abs(exact) > 1e-3
    assert (err[big] / np.abs(exact[big])).max() <= 1e-5


def test_special_values():
    clamp, c = header_constants()
    g = kernel_gelu(np.array([0.0, np.inf, np.nan, 40.0, -40.0], dtype=np.float32), clamp, c)
    assert g[0] == 0.0 and g[1] == np.inf and np.isnan(g[2])
    assert g[3] == np.float32(40.0) and abs(g[4]) < 1e-6
