"""CPU checks of the error-bound helper used by the rotation parity tests."""
import math

import numpy as np

from oracle import ref
from gpu_helpers import abs_butterfly_apply


def test_abs_butterfly_bounds_the_butterfly():
    # |B x| <= |S_{L-1}| ... |S_0| |x| elementwise, both orientations
    rng = np.random.default_rng(5)
    for L in (1, 3, 6):
        n = 1 << L
        a = rng.uniform(-math.pi, math.pi, size=(L, n // 2))
        x = rng.standard_normal((n, 4))
        for tr in (False, True):
            got = np.abs(ref.butterfly_apply(a, x, transpose=tr))
            assert np.all(got <= abs_butterfly_apply(a, np.abs(x), transpose=tr) + 1e-12)


def test_abs_butterfly_single_stage_and_identity():
    # one stage: exactly [[|c|, |s|], [|s|, |c|]] |x|; zero angles: identity
    t = 0.7
    x = np.array([[2.0], [3.0]])
    want = np.array([[abs(math.cos(t)) * 2 + abs(math.sin(t)) * 3],
                     [abs(math.sin(t)) * 2 + abs(math.cos(t)) * 3]])
    np.testing.assert_allclose(abs_butterfly_apply(np.array([[t]]), x), want, rtol=1e-15)
    z = np.zeros((4, 8))
    v = np.random.default_rng(1).random((16, 3))
    np.testing.assert_array_equal(abs_butterfly_apply(z, v), v)
    np.testing.assert_array_equal(abs_butterfly_apply(z, v, transpose=True), v)
