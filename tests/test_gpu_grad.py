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
    # inplace: dx written over dy (True or "dy") or over x ("x")
    out = xd if inplace == "x" else dyd if inplace else None
    dx, dang = bm.butterfly_backward(angd, offd, xd, dyd, transpose, dx=out)
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
    (4, 3, 90, ()),
    (6, 16, 500, (0, 7)),
    (8, 6, 700, (2,)),   # width 256: 32-row LDS tiles, several chunks
    (9, 8, 300, (3,)),
    (10, 5, 120, ()),
    (11, 3, 40, (1,)),
    (12, 3, 9, (0,)),
    (13, 2, 5, ()),
    (7, 4, 1300, ()),    # experts of several chunks
    (9, 4, 40000, (2,)), # width 512, chunks of 64 rows
    (9, 7, 900, (0, 4)), # width 512, 8-row chunks, ragged tails
    (10, 4, 2001, (1,)), # width 1024 in one pass, two rows per step: odd row counts
    (11, 5, 2500, (2,)), # width 2048 in one pass: 16-row chunks, ragged tails
    (12, 4, 700, (1,)),  # width 4096 in part passes: several 32-row chunks, ragged tails
    (13, 3, 150, ()),    # width 8192 in part passes
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
    check_case(12, 2, 90, False, "bf16", seed=6, inplace=True)  # part passes
    check_case(11, 3, 150, True, "f32", seed=8, inplace=True)   # one-pass width 2048
    check_case(10, 3, 77, False, "bf16", seed=9, inplace=True)  # one-pass width 1024
    # dx over x: the one-pass kernels where two or four waves share a row
    # (widths 1024, 2048) and the part passes, whose last pass re-reads x (4096)
    for L, tr, seed in ((10, False, 41), (11, True, 42), (12, False, 43), (13, True, 44)):
        for act in ("f32", "bf16"):
            check_case(L, 3, 130, tr, act, seed=seed + (act == "bf16"), inplace="x")
    # no rows: every expert's angle gradients are zero, no row buffer touched
    ang = torch.randn(3, 5, 16, device="cuda")
    off = torch.zeros(4, dtype=torch.int32, device="cuda")
    x = torch.empty((0, 32), device="cuda")
    dx, dang = bm.butterfly_backward(ang, off, x, x)
    torch.cuda.synchronize()
    assert torch.count_nonzero(dang).item() == 0


def test_expert_angle_gradients_compose():
    # One square expert y = B(phi) (alpha W B(theta)^T x) per bucket of rows:
    # the output rotation's backward gives d phi and dZ, the substrate's
    # transposed product (the ternary GEMM with W^T packed) gives dU, the input
    # rotation's backward gives d theta and dx.  Against the oracle's chain in
    # fp64, and two angles of each rotation against central differences of
    # the oracle's expert.
    import torch
    r = np.random.default_rng(21)
    d, N, R, alpha = 256, 4, 300, 0.5
    L = int(math.log2(d))
    W = r.integers(-1, 2, size=(d, d)).astype(np.int8)
    th = r.uniform(-math.pi, math.pi, size=(N, L, d // 2)).astype(np.float32)
    ph = r.uniform(-math.pi, math.pi, size=(N, L, d // 2)).astype(np.float32)
    off = np.array([0, 90, 90, 210, R], dtype=np.int32)   # expert 1 has no rows
    x = r.standard_normal((R, d)).astype(np.float32)
    dy = r.standard_normal((R, d)).astype(np.float32)
    log("expert angle gradients through the C ABI")
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    xd, dyd, thd, phd, offd = dev(x), dev(dy), dev(th), dev(ph), dev(off)
    Wp = dev(bm.pack_ternary(W).view(np.int32))
    WTp = dev(bm.pack_ternary(np.ascontiguousarray(W.T)).view(np.int32))
    U = torch.empty_like(xd)
    for e in range(N):
        if off[e + 1] > off[e]:
            U[off[e]:off[e + 1]] = bm.dbg_butterfly(thd[e], xd[off[e]:off[e + 1]].contiguous(), transpose=True)
    Z = bm.dbg_ternary_gemm(U, Wp, d, alpha)
    dZ, dph = bm.butterfly_backward(phd, offd, Z, dyd, False)
    dU = bm.dbg_ternary_gemm(dZ, WTp, d, alpha)
    dx, dth = bm.butterfly_backward(thd, offd, xd, dU, True)
    # the substrate's latent gradient (straight-through) from bf16 copies of U and dZ
    U16, dZ16 = U.to(torch.bfloat16), dZ.to(torch.bfloat16)
    dW = bm.substrate_grad(dZ16, U16, alpha)
    torch.cuda.synchronize()
    dWr = ref.substrate_weight_grad(U16.float().cpu().numpy().astype(np.float64),
                                    dZ16.float().cpu().numpy().astype(np.float64), alpha)
    # elementwise against the sum's magnitude |alpha| sqrt(sum_r dZ^2 U^2) (fp32 accumulation)
    u64, dz64 = (t.float().cpu().numpy().astype(np.float64) for t in (U16, dZ16))
    wscale = abs(alpha) * np.sqrt((dz64 ** 2).T @ (u64 ** 2))
    assert np.all(np.abs(dW.cpu().numpy() - dWr) <= 1e-5 * wscale + 1e-30)
    assert np.linalg.norm(dW.cpu().numpy() - dWr) <= 1e-5 * np.linalg.norm(dWr)
    dx, dth, dph = (t.cpu().numpy().astype(np.float64) for t in (dx, dth, dph))
    W64 = W.astype(np.float64)
    for e in range(N):
        r0, r1 = int(off[e]), int(off[e + 1])
        if r1 == r0:
            assert not dth[e].any() and not dph[e].any()
            continue
        X, DY = x[r0:r1].T.astype(np.float64), dy[r0:r1].T.astype(np.float64)
        t64, p64 = th[e].astype(np.float64), ph[e].astype(np.float64)
        Zr = alpha * (W64 @ ref.butterfly_apply(t64, X, transpose=True))
        dZr, dP = ref.butterfly_backward(p64, Zr, DY, False)
        dXr, dT = ref.butterfly_backward(t64, X, alpha * (W64.T @ dZr), True)
        for got, want, what in ((dth[e], dT, "theta"), (dph[e], dP, "phi")):
            rel = np.linalg.norm(got - want) / np.linalg.norm(want)
            assert rel <= 1e-4, f"expert {e} d{what}: {rel:.3g}"
        assert row_rel_err(dx[r0:r1], dXr.T).max() <= 1e-4
        # the chain itself against central differences of the expert
        loss = lambda t, p: float(np.sum(DY * ref.expert_apply(t, p, W64, X, alpha)))
        h = 1e-6
        for (s_, q) in ((0, 3), (L - 1, 100)):
            for which, grad in (("t", dT), ("p", dP)):
                tp, tm, pp, pm = t64.copy(), t64.copy(), p64.copy(), p64.copy()
                if which == "t":
                    tp[s_, q] += h
                    tm[s_, q] -= h
                else:
                    pp[s_, q] += h
                    pm[s_, q] -= h
                fd = (loss(tp, pp) - loss(tm, pm)) / (2 * h)
                assert abs(fd - grad[s_, q]) <= 1e-6 * (1 + abs(fd))
    # the oracle's substrate gradient over all rows (fp64 chain) against central
    # differences of the summed loss of every expert in one substrate entry
    Ur = np.zeros((R, d))
    dZr_all = np.zeros((R, d))
    for e in range(N):
        r0, r1 = int(off[e]), int(off[e + 1])
        if r1 == r0:
            continue
        X = x[r0:r1].T.astype(np.float64)
        Ue = ref.butterfly_apply(th[e].astype(np.float64), X, transpose=True)
        dZe, _ = ref.butterfly_backward(ph[e].astype(np.float64), alpha * (W64 @ Ue), dy[r0:r1].T.astype(np.float64), False)
        Ur[r0:r1], dZr_all[r0:r1] = Ue.T, dZe.T
    dW64 = ref.substrate_weight_grad(Ur, dZr_all, alpha)

    def total_loss(Wm):
        return sum(float(np.sum(dy[off[e]:off[e + 1]].T.astype(np.float64) *
                                ref.expert_apply(th[e].astype(np.float64), ph[e].astype(np.float64), Wm,
                                                 x[off[e]:off[e + 1]].T.astype(np.float64), alpha)))
                   for e in range(N) if off[e + 1] > off[e])
    for (o, i) in ((0, 0), (17, 200), (255, 3)):
        wp, wm = W64.copy(), W64.copy()
        wp[o, i] += 1e-6
        wm[o, i] -= 1e-6
        fd = (total_loss(wp) - total_loss(wm)) / 2e-6
        assert abs(fd - dW64[o, i]) <= 1e-6 * (1 + abs(fd))
