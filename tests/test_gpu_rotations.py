"""GPU parity of each bf16 rotation on its own, inside the production kernels.

The expert is B(phi) W_base B(theta)^T (ButterflyMoE zh page, technical
summary §2.1).  With W_base the identity (a ternary matrix) and the angles of
one side all zero (whose Givens factors are exactly the identity), the layer
reduces to one rotation: y_t = g_t B(phi_e) x_t, or y_t = g_t B(theta_e)^T x_t.
Run through bmoe_forward with prepared weights, every bf16 layer then applies
that single rotation with the kernels the real layers use: the square
expert kernel's two block factors at widths 256 / 512, the low and high parts
at widths 1024 .. 8192, and (FFN layers with identity-embedding substrates)
the FFN middle's B(phi_up) and B(theta_dn)^T.  Angle patterns that are zero
outside the stages of one factor isolate that factor.

Each output element is compared with the oracle's stage-by-stage butterfly
(ref.butterfly_apply) against a forward error bound: with bf16 factor entries
(relative error <= u = 2^-8 each), bf16 rounding of the data after every
factor and fp32 accumulation, |y_i - yhat_i| <= g (c u chain_i + 1e-5 |x|_2)
+ u |yhat_i|, where chain = |S_{L-1}| ... |S_0| |x| is the butterfly applied
with |cos| and |sin| (it bounds |G_k| ... |G_1| |x| elementwise, the G being
products of stages) and c counts the factor entries and roundings on the path.
"""
import math

import numpy as np
import pytest

import compressed_mixture_experts_amd as bm
from compressed_mixture_experts_amd import workloads as wl
from oracle import ref
from gpu_helpers import abs_butterfly_apply, log, run_layer, to_f64

pytestmark = pytest.mark.gpu

U = 2.0 ** -8


@pytest.fixture(scope="module", autouse=True)
def _cuda():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    bm.lib()
    yield


def _angle_pattern(rng, n_experts, n, part, split_at):
    """Angles [N][L][n/2]: uniform in the stages of `part` ("all", "low":
    stages below split_at, "high": stages from split_at on), zero elsewhere."""
    L = int(math.log2(n))
    a = rng.uniform(-math.pi, math.pi, size=(n_experts, L, n // 2))
    if part == "low":
        a[:, split_at:] = 0.0
    elif part == "high":
        a[:, :split_at] = 0.0
    return np.ascontiguousarray(a, dtype=np.float32)


def _factor_split(n):
    """Stage index where the kernels' second factor starts: the square expert
    kernel's 32- / 16-index blocks at widths 512 / 256, the low / high parts
    (low = stages 0 .. L-5) at widths 1024 .. 8192."""
    L = int(math.log2(n))
    return {8: 4, 9: 5}.get(L, L - 4)


def _check(y_gpu, want, chain, x_norm, g, c):
    bound = g[:, None] * (c * U * chain + 1e-5 * x_norm[:, None]) + U * np.abs(want)
    diff = np.abs(y_gpu - want)
    worst = (diff / bound).max()
    log(f"  max |err| {diff.max():.3e}, worst err/bound {worst:.3f}")
    assert np.all(diff <= bound), worst


# (width, tokens): several expert tiles and a ragged tail at every width
SQUARE = [(256, 300), (512, 300), (1024, 260), (2048, 200), (4096, 150), (8192, 100)]


@pytest.mark.parametrize("side", ["phi", "theta"])
@pytest.mark.parametrize("part", ["all", "low", "high"])
@pytest.mark.parametrize("n,T", SQUARE)
def test_square_layer_single_rotation(n, T, part, side):
    N = 3
    cfg = wl.small_config(d_model=n, n_experts=N, top_k=1, tokens=T, act="bf16", seed_index=600 + n % 97)
    inp = wl.generate(cfg)
    rng = np.random.default_rng(n + (7 if side == "theta" else 0) + {"all": 0, "low": 1, "high": 2}[part])
    ang = _angle_pattern(rng, N, n, part, _factor_split(n))
    zero = np.zeros_like(ang)
    inp.w_base[0] = np.eye(n, dtype=np.int8)
    inp.theta[0], inp.phi[0] = (ang, zero) if side == "theta" else (zero, ang)
    log(f"single rotation: square n={n} T={T} {side} stages={part}")
    _, _, (y, idx, gate) = run_layer(inp, prepared=True)
    idx = idx.cpu().numpy()[:, 0]
    g = gate.cpu().numpy().astype(np.float64)[:, 0]
    x = ref.stored_to_f64(inp.x, "bf16")
    R = ref.route(x, ref.stored_to_f64(inp.w_gate, "bf16"), 1)
    assert np.array_equal(idx, R.idx[:, 0])
    want = np.empty_like(x)
    chain = np.empty_like(x)
    for e in range(N):
        t = np.nonzero(idx == e)[0]
        if not len(t):
            continue
        tr = side == "theta"
        want[t] = ref.butterfly_apply(ang[e], x[t].T, transpose=tr).T * R.gates[t, :1]
        chain[t] = abs_butterfly_apply(ang[e], np.abs(x[t]).T, transpose=tr).T
    # three bf16 factor entries and three roundings on a path (two at 256 / 512), plus the gate
    _check(to_f64(y), want, chain, np.linalg.norm(x, axis=1), g, 8.0)


@pytest.mark.parametrize("n,side", [(1024, "phi"), (1024, "theta"), (2048, "phi"), (2048, "theta")])
def test_square_layer_single_rotation_tall_tiles(n, side):
    # 33000 routed rows at widths 1024 / 2048: the one-pass rotations take
    # 64-row workgroups that keep every factor in registers over four 16-row
    # sub-tiles (three experts: tiles of 64 with ragged ends)
    T, N = 33000, 3
    cfg = wl.small_config(d_model=n, n_experts=N, top_k=1, tokens=T, act="bf16", seed_index=640)
    inp = wl.generate(cfg)
    rng = np.random.default_rng(n + (7 if side == "theta" else 0))
    ang = _angle_pattern(rng, N, n, "all", 0)
    zero = np.zeros_like(ang)
    inp.w_base[0] = np.eye(n, dtype=np.int8)
    inp.theta[0], inp.phi[0] = (ang, zero) if side == "theta" else (zero, ang)
    log(f"single rotation, tall tiles: square n={n} T={T} {side}")
    _, _, (y, idx, gate) = run_layer(inp, prepared=True)
    idx = idx.cpu().numpy()[:, 0]
    g = gate.cpu().numpy().astype(np.float64)[:, 0]
    x = ref.stored_to_f64(inp.x, "bf16")
    R = ref.route(x, ref.stored_to_f64(inp.w_gate, "bf16"), 1)
    assert np.array_equal(idx, R.idx[:, 0])
    want = np.empty_like(x)
    chain = np.empty_like(x)
    for e in range(N):
        t = np.nonzero(idx == e)[0]
        if not len(t):
            continue
        tr = side == "theta"
        want[t] = ref.butterfly_apply(ang[e], x[t].T, transpose=tr).T * R.gates[t, :1]
        chain[t] = abs_butterfly_apply(ang[e], np.abs(x[t]).T, transpose=tr).T
    _check(to_f64(y), want, chain, np.linalg.norm(x, axis=1), g, 8.0)


# FFN middle: W_up = [I; 0] (d_ff x d), W_dn = [I 0] (d x d_ff), theta_up = phi_dn = 0,
# no activation: y_t = g_t [I 0] B(theta_dn)^T B(phi_up) [x_t; 0]
FFN = [(256, 1024, 200), (256, 4096, 120), (256, 8192, 80)]


@pytest.mark.parametrize("which", ["phi_up", "theta_dn", "both"])
@pytest.mark.parametrize("d,f,T", FFN)
def test_ffn_middle_rotations(d, f, T, which):
    N = 3
    cfg = wl.small_config(d_model=d, d_ff=f, n_experts=N, top_k=1, tokens=T, act="bf16",
                          ffn_act="none", seed_index=700 + f % 89)
    inp = wl.generate(cfg)
    rng = np.random.default_rng(f + {"phi_up": 0, "theta_dn": 1, "both": 2}[which])
    a_up = _angle_pattern(rng, N, f, "all", 0)
    a_dn = _angle_pattern(rng, N, f, "all", 0)
    if which == "phi_up":
        a_dn[:] = 0.0
    elif which == "theta_dn":
        a_up[:] = 0.0
    inp.w_base[0] = np.eye(f, d, dtype=np.int8)
    inp.w_base[1] = np.eye(d, f, dtype=np.int8)
    inp.theta[0] = np.zeros_like(inp.theta[0])
    inp.phi[1] = np.zeros_like(inp.phi[1])
    inp.phi[0], inp.theta[1] = a_up, a_dn
    log(f"single rotation: FFN middle d={d} d_ff={f} T={T} {which}")
    _, _, (y, idx, gate) = run_layer(inp, prepared=True)
    idx = idx.cpu().numpy()[:, 0]
    g = gate.cpu().numpy().astype(np.float64)[:, 0]
    x = ref.stored_to_f64(inp.x, "bf16")
    R = ref.route(x, ref.stored_to_f64(inp.w_gate, "bf16"), 1)
    assert np.array_equal(idx, R.idx[:, 0])
    want = np.empty_like(x)
    chain = np.empty_like(x)
    for e in range(N):
        t = np.nonzero(idx == e)[0]
        if not len(t):
            continue
        h = np.zeros((f, len(t)))
        h[:d] = x[t].T
        v = ref.butterfly_apply(a_dn[e], ref.butterfly_apply(a_up[e], h), transpose=True)
        want[t] = v[:d].T * R.gates[t, :1]
        ha = np.zeros((f, len(t)))
        ha[:d] = np.abs(x[t]).T
        ca = abs_butterfly_apply(a_dn[e], abs_butterfly_apply(a_up[e], ha), transpose=True)
        chain[t] = ca[:d].T
    # up to six factor entries and six roundings on a path, plus the gate
    _check(to_f64(y), want, chain, np.linalg.norm(x, axis=1), g, 14.0)

