"""GPU parity of the butterfly backward (include/bmoe_grad.h) against the fp64
oracle's chain rule (oracle.ref.butterfly_backward, pinned by finite
differences in test_oracle_pins.py).

Rows are bucketed by expert with some experts empty.  Bars: input gradients
per-row relative L2 <= 2e-5 (fp32 rows; fp32 arithmetic over at most 13
stages) or <= 8e-3 (bf16 rows: the output rounding, 2^-9 per element, plus
the same arithmetic); angle gradients per expert ||d - ref|| / ||ref|| <= 1e-4
(fp32 sums over the expert's rows), exactly zero for an expert without rows.
"""
import math

import numpy as np
import pytest

import compressed_mixture_experts_amd as bm
from compressed_mixture_experts_amd import workloads as wl
from oracle import ref
from gpu_helpers import log, row_rel_err, to_dev, to_f64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _cuda():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    bm.lib()
    yield


def make_case(L, N, rows, act, seed, empty=()):
    r = np.random.default_rng(seed)
    n = 1 << L
    ang = r.uniform(-math.pi, math.pi, size=(N, L, n // 2)).astype(np.float32)
    w = r.uniform(0.2, 1.0, size=N)
    for e in empty:
        w[e] = 0.0
    cnt = np.floor(rows * w / w.sum()).astype(int)
    cnt[int(np.argmax(w))] += rows - cnt.sum()
    off = np.concatenate([[0], np.cumsum(cnt)]).astype(np.int32)
    x = wl._store(r.standard_normal((rows, n)), act)
    dy = wl._store(r.standard_normal((rows, n)), act)
    return ang, off, x, dy


def check_case(L, N, rows, transpose, act, seed, empty=(), inplace=False):
    import torch
    ang, off, x, dy = make_case(L, N, rows, act, seed, empty)
    log(f"butterfly backward L={L} N={N} rows={rows} transpose={transpose} act={act} inplace={inplace}")
    xd, dyd = to_dev(x, act), to_dev(dy, act)
    angd = torch.from_numpy(ang).cuda()
    offd = torch.from_numpy(off).cuda()
    dx, dang = bm.butterfly_backward(angd, offd, xd, dyd, transpose, dx=dyd if inplace else None)
    torch.cuda.synchronize()
    dx, dang = to_f64(dx), dang.cpu().numpy().astype(np.float64)
    x64, dy64 = ref.stored_to_f64(x, act), ref.stored_to_f64(dy, act)
    tol_x = 2e-5 if act == "f32" else 8e-3
    for e in range(N):
        r0, r1 = int(off[e]), int(off[e + 1])
        if r1 == r0:
            assert np.all(dang[e] == 0.0), f"expert {e} has no rows but nonzero angle gradients"
            continue
        dX, dA = ref.butterfly_backward(ang[e].astype(np.float64), x64[r0:r1].T, dy64[r0:r1].T, transpose)
        if (r1 - r0) << L > (1 << 22):
            log(f"  expert {e}: {r1 - r0} rows checked")
        err = row_rel_err(dx[r0:r1], dX.T)
        assert err.max() <= tol_x, f"expert {e}: dx row error {err.max():.3g}"
        rel = np.linalg.norm(dang[e] - dA) / max(np.linalg.norm(dA), 1e-30)
        assert rel <= 1e-4, f"expert {e}: angle gradient error {rel:.3g}"


CASES = [
    # (L, N, rows, empty experts)
    (1, 3, 20, (1,)),
    (3, 4, 50, ()),
    (6, 16, 500, (0, 7)),
    (9, 8, 300, (3,)),
    (10, 5, 120, ()),
    (11, 3, 40, (1,)),
    (12, 3, 9, (0,)),
    (13, 2, 5, ()),
    (7, 4, 1300, ()),    # experts of several chunks
    (9, 4, 40000, (2,)), # chunks of two 32-row sub-tiles
]


@pytest.mark.parametrize("case", range(len(CASES)))
@pytest.mark.parametrize("transpose", [False, True])
@pytest.mark.parametrize("act", ["f32", "bf16"])
def test_butterfly_backward(case, transpose, act):
    L, N, rows, empty = CASES[case]
    check_case(L, N, rows, transpose, act, seed=31 * case + 7 * transpose + (act == "bf16"), empty=empty)


def test_butterfly_backward_wide_chunks():
    # width 8192 with chunks of two 2-row sub-tiles (one orientation and dtype:
    # the fp64 check of 2100 rows of 8192 takes most of a minute)
    check_case(13, 2, 2100, True, "bf16", seed=77)


def test_butterfly_backward_in_place_and_zero_rows():
    import torch
    check_case(9, 4, 130, True, "f32", seed=5, inplace=True)
    # no rows: every expert's angle gradients are zero, no row buffer touched
    ang = torch.randn(3, 5, 16, device="cuda")
    off = torch.zeros(4, dtype=torch.int32, device="cuda")
    x = torch.empty((0, 32), device="cuda")
    dx, dang = bm.butterfly_backward(ang, off, x, x)
    torch.cuda.synchronize()
    assert torch.count_nonzero(dang).item() == 0
