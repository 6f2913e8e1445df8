"""GPU parity of the substrate's weight gradient (include/bmoe_grad.h,
bmoe_substrate_grad) against the fp64 oracle (oracle.ref.substrate_weight_grad,
pinned by central differences of the substrate product in test_oracle_pins.py).

Inputs are bf16 (the oracle reads the same bf16 values), so the only error is
the fp32 accumulation over the rows: the bar is, per output, |d - ref| <=
1e-5 * sqrt(sum_r (dz[r][o] u[r][i])^2) + 1e-30, and the relative Frobenius
error <= 1e-5.  At the full large-workload shape the check samples outputs
(each an fp64 dot product over all rows).
"""
import numpy as np
import pytest

import compressed_mixture_experts_amd as bm
from oracle import ref
from gpu_helpers import log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _cuda():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    bm.lib()
    yield


def _bf16_rows(r, rows, d, scale=1.0):
    import torch
    return (torch.from_numpy(r.standard_normal((rows, d)).astype(np.float32)) * scale).to(torch.bfloat16)


def _f64(t):
    import torch
    return t.to(torch.float32).numpy().astype(np.float64)


@pytest.mark.parametrize("rows,d_out,d_in,alpha", [
    (300, 128, 256, 1.0),      # one split, ragged last step (300 = 9 x 32 + 12)
    (16384, 512, 512, 0.5),    # edge workload: T k rows, split over the rows
    (5000, 1024, 384, -2.0),   # ragged split lengths, non-square
    (33, 256, 128, 1.0),       # fewer rows than one step beyond the first
    (1, 128, 128, 3.0),
    (300, 4096, 4096, 1.0),    # 256 x 256 output tiles (eight waves), ragged last step
])
def test_substrate_grad_matches_oracle(rows, d_out, d_in, alpha):
    import torch
    r = np.random.default_rng(rows + d_out)
    log(f"substrate grad rows={rows} d_out={d_out} d_in={d_in} alpha={alpha}")
    dz, u = _bf16_rows(r, rows, d_out), _bf16_rows(r, rows, d_in)
    dw = bm.substrate_grad(dz.cuda(), u.cuda(), alpha)
    torch.cuda.synchronize()
    got = dw.cpu().numpy().astype(np.float64)
    dz64, u64 = _f64(dz), _f64(u)
    want = ref.substrate_weight_grad(u64, dz64, alpha)
    scale = abs(alpha) * np.sqrt((dz64 ** 2).T @ (u64 ** 2))
    assert np.all(np.abs(got - want) <= 1e-5 * scale + 1e-30), np.max(np.abs(got - want) / (scale + 1e-30))
    assert np.linalg.norm(got - want) <= 1e-5 * np.linalg.norm(want)


def test_substrate_grad_zero_rows_and_repeat():
    import torch
    dw = torch.full((256, 128), 7.0, device="cuda")
    empty = torch.empty((0, 256), dtype=torch.bfloat16, device="cuda")
    bm.substrate_grad(empty, torch.empty((0, 128), dtype=torch.bfloat16, device="cuda"), 1.0, dw=dw)
    torch.cuda.synchronize()
    assert torch.count_nonzero(dw).item() == 0
    # the same call twice gives the same bits (splits added in order)
    r = np.random.default_rng(3)
    dz, u = _bf16_rows(r, 9000, 512).cuda(), _bf16_rows(r, 9000, 512).cuda()
    a = bm.substrate_grad(dz, u, 1.0)
    b = bm.substrate_grad(dz, u, 1.0)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_substrate_grad_large_shape_sampled():
    # the large workload's FFN up substrate: 65536 routed rows, d_out 8192,
    # d_in 2048 (no split); 64 sampled outputs, each an fp64 dot product
    import torch
    rows, d_out, d_in = 65536, 8192, 2048
    log(f"substrate grad sampled rows={rows} d_out={d_out} d_in={d_in}")
    g = torch.Generator(device="cuda").manual_seed(5)
    dz = torch.randn((rows, d_out), device="cuda", generator=g).to(torch.bfloat16)
    u = torch.randn((rows, d_in), device="cuda", generator=g).to(torch.bfloat16)
    dw = bm.substrate_grad(dz, u, 0.25)
    torch.cuda.synchronize()
    r = np.random.default_rng(9)
    os_ = r.integers(0, d_out, 64)
    is_ = r.integers(0, d_in, 64)
    dzc = dz[:, torch.from_numpy(os_).cuda()].float().cpu().numpy().astype(np.float64)
    uc = u[:, torch.from_numpy(is_).cuda()].float().cpu().numpy().astype(np.float64)
    got = dw[torch.from_numpy(os_).cuda(), torch.from_numpy(is_).cuda()].cpu().numpy().astype(np.float64)
    want = 0.25 * np.sum(dzc * uc, axis=0)
    scale = 0.25 * np.sqrt(np.sum((dzc * uc) ** 2, axis=0))
    assert np.all(np.abs(got - want) <= 1e-5 * scale), np.max(np.abs(got - want) / scale)
