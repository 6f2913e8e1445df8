"""Host checks of the outlier-spread statistics bench.py reports (peak-to-RMS
ratio and ternary-code error), on rows whose values follow by hand."""
import math

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import bench


def test_spread_stats_hand_values():
    # row [3, 0, 0, 4]: rms 2.5, peak 4 -> 1.6; mean|v| 1.75, threshold 1.225
    # keeps {3, 4}, a = 3.5, code [3.5, 0, 0, 3.5], error (0.25 + 0.25) / 25
    p, e = bench.spread_stats(torch.tensor([[3.0, 0.0, 0.0, 4.0]]))
    assert p == pytest.approx(1.6)
    assert e == pytest.approx(0.02)


def test_spread_stats_spike_and_flat():
    # a single spike in n entries: peak sqrt(n), coded exactly; a flat row
    # of +-1: peak 1, coded exactly
    n = 64
    spike = torch.zeros(1, n)
    spike[0, 5] = -2.0
    p, e = bench.spread_stats(spike)
    assert p == pytest.approx(math.sqrt(n))
    assert e == pytest.approx(0.0, abs=1e-12)
    flat = torch.from_numpy(np.where(np.arange(n) % 3 == 0, -1.0, 1.0)[None, :].astype(np.float32))
    p, e = bench.spread_stats(flat)
    assert p == pytest.approx(1.0)
    assert e == pytest.approx(0.0, abs=1e-12)
