"""Coefficients of the GELU used by the FFN middle kernels (butterfly_impl.hpp).

GELU(h) = h Phi(h) = relu(h) - |h| Q(|h|), with Q(a) = Phi(-a) = erfc(a / sqrt 2) / 2
the upper normal tail.  log2 Q(a) is smooth on [0, A] (A = 5.75, where Q is about
4.5e-9), so the kernels evaluate a polynomial P(a) of degree 7 there and take
Q = exp2(P(min(|h|, A))): one hardware exp2, seven FMAs, no reciprocal (the clamp is one med3).

The polynomial is a minimax fit of log2 Q in the absolute sense (relative error
of Q), by Lawson's iteratively reweighted least squares over Chebyshev nodes,
in the variable a / A and converted to powers of a.  Run this file to print the
constants; tests/test_gelu_tail.py checks the printed values against the header
and the resulting GELU against the exact one.
"""
import numpy as np
from scipy.special import log_ndtr

A = 5.75
DEGREE = 7


def fit(degree: int = DEGREE, nodes: int = 4000, iters: int = 60) -> np.ndarray:
    k = np.arange(nodes)
    x = 0.5 - 0.5 * np.cos(np.pi * (k + 0.5) / nodes)
    y = log_ndtr(-A * x) / np.log(2.0)
    V = np.vander(x, degree + 1, increasing=True)
    w = np.ones_like(x)
    c = None
    for _ in range(iters):
        c, *_ = np.linalg.lstsq(V * np.sqrt(w)[:, None], y * np.sqrt(w), rcond=None)
        r = np.abs(V @ c - y)
        w = np.maximum(w * r / np.mean(w * r), 1e-12)
    return (c / A ** np.arange(degree + 1)).astype(np.float32)   # powers of a


if __name__ == "__main__":
    for i, v in enumerate(fit()):
        print(f"  {float(v):.9e}f,  // a^{i}")
