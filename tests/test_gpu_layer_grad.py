"""GPU backward of a whole routed square layer composed from the C ABI, against
the fp64 oracle (oracle.ref.layer_backward_experts, pinned by central
differences of the oracle's layer forward in test_oracle_pins.py).

Routing and gates are held at the router's choice.  Pieces: bmoe_route
(buckets), the input rotation, the ternary substrate product and the output
rotation for the forward values; bmoe_combine_backward (gradient at each
routed row, gate gradients); bmoe_butterfly_backward through the output
rotation (dphi, dZ); the substrate product with W^T packed (dU);
bmoe_butterfly_backward through the input rotation (dtheta, per-row dx);
bmoe_substrate_grad (dW, bf16 copies of U and dZ).  Per-row input gradients
are added into tokens by the test itself.  Bars, elementwise: fp32 rows;
angle gradients and dx within 3e-5 of (|ref| + the expert's or token's RMS),
gate gradients within 1e-4 of |dy||o|, dW within 2^-7 alpha sum |dZ|^T |U|
(its inputs rounded to bf16: one rounding each).
"""
import math

import numpy as np
import pytest

import compressed_mixture_experts_amd as bm
from compressed_mixture_experts_amd import workloads as wl
from oracle import ref
from gpu_helpers import log, row_rel_err

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _cuda():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    bm.lib()
    yield


def test_combine_backward_matches_definition():
    import torch
    r = np.random.default_rng(2)
    T, k, d = 700, 2, 256
    for act in ("f32", "bf16"):
        log(f"combine backward act={act}")
        dt = torch.float32 if act == "f32" else torch.bfloat16
        dy = torch.from_numpy(r.standard_normal((T, d)).astype(np.float32)).to(dt).cuda()
        o = torch.from_numpy(r.standard_normal((T * k, d)).astype(np.float32)).to(dt).cuda()
        slots = torch.from_numpy(r.permutation(T * k).astype(np.int32)).cuda()
        gate = torch.from_numpy(r.uniform(0, 1, T * k).astype(np.float32)).cuda()
        d_rows, d_gate = bm.combine_backward(dy, slots, gate, k, o)
        d_rows2, none = bm.combine_backward(dy, slots, gate, k)
        torch.cuda.synchronize()
        assert none is None and torch.equal(d_rows, d_rows2)
        s = slots.cpu().numpy()
        dy64 = dy.float().cpu().numpy().astype(np.float64)
        o64 = o.float().cpu().numpy().astype(np.float64)
        g = gate.cpu().numpy()
        want = (g[s][:, None].astype(np.float32) * dy.float().cpu().numpy()[s // k])  # one fp32 product
        got = d_rows.float().cpu().numpy()
        if act == "f32":
            assert np.array_equal(got, want)
        else:
            assert np.all(np.abs(got - want) <= np.abs(want) * 2.0 ** -8)
        wg = np.sum(dy64[s // k] * o64, axis=1)
        scale = np.linalg.norm(dy64[s // k], axis=1) * np.linalg.norm(o64, axis=1)
        assert np.all(np.abs(d_gate.cpu().numpy()[s] - wg) <= 1e-5 * scale)


def test_layer_backward_composed_from_the_abi():
    import torch
    cfg = wl.small_config(d_model=256, n_experts=6, top_k=2, tokens=600, act="f32", w_scale=0.5, seed_index=17)
    inp = wl.generate(cfg)
    x64 = ref.stored_to_f64(inp.x, "f32")
    R = ref.route(x64, ref.stored_to_f64(inp.w_gate, "f32"), cfg.top_k)
    layer = bm.Layer.from_inputs(inp)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    x = dev(inp.x)
    log("layer backward: route")
    idx, gate, off, slots = layer.route(x, with_buckets=True)
    torch.cuda.synchronize()
    same = (idx.cpu().numpy() == R.idx).all(axis=1)
    assert same.all(), "routing differs from the oracle (pick a seed without near ties)"
    k, d, N, alpha = cfg.top_k, cfg.d_model, cfg.n_experts, cfg.w_scale
    L = int(math.log2(d))
    offs = off.cpu().numpy()
    th = dev(inp.theta[0].astype(np.float32))
    ph = dev(inp.phi[0].astype(np.float32))
    W = inp.w_base[0]
    Wp = dev(bm.pack_ternary(W).view(np.int32))
    WTp = dev(bm.pack_ternary(np.ascontiguousarray(W.T)).view(np.int32))
    tok = (slots // k).long()
    xb = x[tok].contiguous()                      # rows in bucket order
    U = torch.empty_like(xb)
    for e in range(N):
        if offs[e + 1] > offs[e]:
            U[offs[e]:offs[e + 1]] = bm.dbg_butterfly(th[e], xb[offs[e]:offs[e + 1]].contiguous(), transpose=True)
    Z = bm.dbg_ternary_gemm(U, Wp, d, alpha)
    O = torch.empty_like(Z)
    for e in range(N):
        if offs[e + 1] > offs[e]:
            O[offs[e]:offs[e + 1]] = bm.dbg_butterfly(ph[e], Z[offs[e]:offs[e + 1]].contiguous(), transpose=False)
    r = np.random.default_rng(5)
    dy64 = r.standard_normal((cfg.tokens, d))
    dy = dev(dy64.astype(np.float32))
    log("layer backward: combine, rotations, substrate")
    gate_flat = gate.reshape(-1).contiguous()
    d_rows, d_gate = bm.combine_backward(dy, slots, gate_flat, k, O)
    dZ, dph = bm.butterfly_backward(ph, off, Z, d_rows, False)
    dU = bm.substrate_input_grad(dZ, WTp, d, alpha)
    dxb, dth = bm.butterfly_backward(th, off, xb, dU, True)
    dW = bm.substrate_grad(dZ.to(torch.bfloat16), U.to(torch.bfloat16), alpha)
    dx = torch.zeros_like(x).index_add_(0, tok, dxb)
    torch.cuda.synchronize()

    want = ref.layer_backward_experts(inp, dy64.astype(np.float32).astype(np.float64), R)
    got_th, got_ph = dth.cpu().numpy(), dph.cpu().numpy()
    # elementwise: within 3e-5 of |ref| + the expert's RMS (fp32 chain rule)
    for got, ref_, what in ((got_th, want["theta"], "theta"), (got_ph, want["phi"], "phi")):
        rms = np.sqrt(np.mean(ref_ ** 2, axis=(1, 2), keepdims=True))
        assert np.all(np.abs(got - ref_) <= 3e-5 * (np.abs(ref_) + rms)), f"d{what}"
    dxw = want["x"]
    dxg = dx.cpu().numpy().astype(np.float64)
    assert np.all(np.abs(dxg - dxw) <= 3e-5 * (np.abs(dxw) + np.sqrt(np.mean(dxw ** 2, axis=1, keepdims=True))))
    dgate = d_gate.cpu().numpy().reshape(cfg.tokens, k)
    ob = np.linalg.norm(dy64, axis=1)[:, None] * np.abs(want["gate"]).max()
    assert np.all(np.abs(dgate - want["gate"]) <= 1e-4 * (1 + ob))
    # dW from bf16 copies of dZ and U: one rounding each, 2^-8 relative per product term
    dWr = want["w_base"]
    assert np.all(np.abs(dW.cpu().numpy() - dWr) <= 2.0 ** -7 * want["w_base_abs"] + 1e-6 * np.abs(dWr).max())
    # the router's part, fed with the GPU's gate gradients: the whole layer's
    # input gradient and the gate matrix's gradient
    wgd = dev(inp.w_gate)
    dx_r, dwg = bm.router_backward(x, wgd, idx, d_gate.reshape(cfg.tokens, k).contiguous(), False)
    torch.cuda.synchronize()
    rdx, rdwg, _ = ref.router_backward(x64, ref.stored_to_f64(inp.w_gate, "f32"), R.idx, want["gate"])
    tot = dx.cpu().numpy().astype(np.float64) + dx_r.cpu().numpy()
    assert row_rel_err(tot, want["x"] + rdx).max() <= 1e-4
    assert np.linalg.norm(dwg.cpu().numpy() - rdwg) <= 1e-4 * np.linalg.norm(rdwg)
    # elementwise, against |ref| + the expert row's RMS (the gate gradients fed
    # in carry their own 1e-4 relative error)
    gw = dwg.cpu().numpy().astype(np.float64)
    rms = np.sqrt(np.mean(rdwg ** 2, axis=1, keepdims=True))
    err = np.abs(gw - rdwg) / (np.abs(rdwg) + rms)
    log(f"  dW_g elementwise: max {err.max():.2e}")
    assert err.max() <= 3e-4


@pytest.mark.parametrize("T,d,N,k,renorm,act", [
    (777, 128, 16, 4, False, "f32"),
    (777, 128, 16, 4, True, "bf16"),
    (4096, 512, 64, 2, False, "bf16"),    # edge workload's router
    (3000, 512, 256, 2, True, "f32"),
    (300, 2048, 256, 2, False, "bf16"),   # large workload's width, several column blocks
    (5, 8, 3, 1, False, "f32"),           # fewer tokens than a tile
    (16500, 256, 64, 2, False, "bf16"),   # 64-token tiles of the dx pass, ragged last tile; 32-token logits tiles
    (33000, 64, 16, 2, True, "bf16"),     # 64-token logits tiles, ragged last tile, one expert block
    (50, 40, 5, 2, False, "bf16"),        # width not a multiple of 32: logits on the VALU
])
def test_router_backward_matches_oracle(T, d, N, k, renorm, act):
    import torch
    r = np.random.default_rng(T + d + N)
    log(f"router backward T={T} d={d} N={N} k={k} renorm={renorm} act={act}")
    x = wl._store(r.standard_normal((T, d)), act)
    wg = wl._store(r.standard_normal((N, d)) / math.sqrt(d), act)
    idx = np.argsort(r.random((T, N)), axis=1)[:, :k].astype(np.int32)   # distinct experts per token
    dgate = r.standard_normal((T, k)).astype(np.float32)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    xd = dev(x) if act == "f32" else dev(x.view(np.int16)).view(torch.bfloat16)
    wd = dev(wg) if act == "f32" else dev(wg.view(np.int16)).view(torch.bfloat16)
    dx, dwg = bm.router_backward(xd, wd, dev(idx), dev(dgate), renorm)
    torch.cuda.synchronize()
    x64, w64 = ref.stored_to_f64(x, act), ref.stored_to_f64(wg, act)
    rdx, rdw, _ = ref.router_backward(x64, w64, idx, dgate.astype(np.float64), renorm)
    got_dx, got_dw = dx.cpu().numpy().astype(np.float64), dwg.cpu().numpy().astype(np.float64)
    scale_x = np.linalg.norm(rdx, axis=1).max()
    assert np.abs(got_dx - rdx).max() <= 1e-4 * scale_x
    # elementwise, against |ref| + the expert row's RMS
    rms = np.sqrt(np.mean(rdw ** 2, axis=1, keepdims=True))
    assert np.all(np.abs(got_dw - rdw) <= 1e-4 * (np.abs(rdw) + rms))


def test_router_backward_zero_tokens():
    import torch
    wd = torch.randn((8, 64), device="cuda")
    dwg = torch.full((8, 64), 3.0, device="cuda")
    x = torch.empty((0, 64), device="cuda")
    idx = torch.empty((0, 2), dtype=torch.int32, device="cuda")
    dg = torch.empty((0, 2), device="cuda")
    dx, dwg = bm.router_backward(x, wd, idx, dg)
    torch.cuda.synchronize()
    assert torch.count_nonzero(dwg).item() == 0 and dx.shape == (0, 64)


def test_gelu_backward_matches_oracle():
    import torch
    r = np.random.default_rng(12)
    for act in ("f32", "bf16"):
        h = wl._store(3.0 * r.standard_normal((300, 256)), act)
        da = wl._store(r.standard_normal((300, 256)), act)
        dev = lambda a: (torch.from_numpy(np.ascontiguousarray(a)).cuda() if act == "f32"
                         else torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16))
        hd, dad = dev(h), dev(da)
        dh = bm.gelu_backward(hd, dad)
        dh2 = bm.gelu_backward(hd, dad.clone(), dh=None)
        inplace = dad.clone()
        bm.gelu_backward(hd, inplace, dh=inplace)
        torch.cuda.synchronize()
        want = ref.gelu_backward(ref.stored_to_f64(h, act), ref.stored_to_f64(da, act))
        got = dh.float().cpu().numpy().astype(np.float64)
        # fp32 arithmetic (the erf approximation within 1.5e-7), then for bf16
        # the output's rounding: half a step, 2^-8 of the result at most
        rnd = 2.0 ** -8 if act == "bf16" else 0.0
        assert np.all(np.abs(got - want) <= rnd * np.abs(want) + 2e-6 * np.abs(ref.stored_to_f64(da, act)) + 1e-30)
        assert torch.equal(dh, dh2) and torch.equal(dh, inplace)


def test_ffn_layer_backward_composed_from_the_abi():
    # the FFN form: route -> (input rotation, up substrate, up rotation, GELU,
    # down input rotation, down substrate, output rotation) forward values ->
    # combine backward -> each piece's backward in reverse, GELU's derivative
    # between the two substrates; against the oracle's FFN backward
    import torch
    cfg = wl.small_config(d_model=128, d_ff=256, n_experts=4, top_k=2, tokens=300, act="f32", w_scale=0.5,
                          seed_index=19)
    inp = wl.generate(cfg)
    x64 = ref.stored_to_f64(inp.x, "f32")
    R = ref.route(x64, ref.stored_to_f64(inp.w_gate, "f32"), cfg.top_k)
    layer = bm.Layer.from_inputs(inp)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    x = dev(inp.x)
    log("ffn layer backward: route")
    idx, gate, off, slots = layer.route(x, with_buckets=True)
    torch.cuda.synchronize()
    assert (idx.cpu().numpy() == R.idx).all(), "routing differs from the oracle (pick a seed without near ties)"
    k, d, f, N, alpha = cfg.top_k, cfg.d_model, cfg.d_ff, cfg.n_experts, cfg.w_scale
    offs = off.cpu().numpy()
    thu, phu = dev(inp.theta[0].astype(np.float32)), dev(inp.phi[0].astype(np.float32))
    thd, phd = dev(inp.theta[1].astype(np.float32)), dev(inp.phi[1].astype(np.float32))
    Wu, Wd = inp.w_base[0], inp.w_base[1]          # [f][d], [d][f]
    pk = lambda W: dev(bm.pack_ternary(np.ascontiguousarray(W)).view(np.int32))
    Wup, WupT, Wdp, WdpT = pk(Wu), pk(Wu.T), pk(Wd), pk(Wd.T)
    tok = (slots // k).long()
    xb = x[tok].contiguous()

    def per_expert(ang, rows, transpose):
        out = torch.empty_like(rows)
        for e in range(N):
            if offs[e + 1] > offs[e]:
                out[offs[e]:offs[e + 1]] = bm.dbg_butterfly(ang[e], rows[offs[e]:offs[e + 1]].contiguous(),
                                                            transpose=transpose)
        return out

    U = per_expert(thu, xb, True)
    H1 = bm.dbg_ternary_gemm(U, Wup, f, alpha)
    H = per_expert(phu, H1, False)
    A = torch.nn.functional.gelu(H, approximate="none")
    V = per_expert(thd, A, True)
    Z = bm.dbg_ternary_gemm(V, Wdp, d, alpha)
    O = per_expert(phd, Z, False)
    dy64 = np.random.default_rng(6).standard_normal((cfg.tokens, d))
    dy = dev(dy64.astype(np.float32))
    log("ffn layer backward: pieces")
    d_rows, d_gate = bm.combine_backward(dy, slots, gate.reshape(-1).contiguous(), k, O)
    dZ, dphd = bm.butterfly_backward(phd, off, Z, d_rows, False)
    dV = bm.substrate_input_grad(dZ, WdpT, f, alpha)
    dA, dthd = bm.butterfly_backward(thd, off, A, dV, True)
    dH = bm.gelu_backward(H, dA)
    dH1, dphu = bm.butterfly_backward(phu, off, H1, dH, False)
    dU = bm.substrate_input_grad(dH1, WupT, d, alpha)
    dxb, dthu = bm.butterfly_backward(thu, off, xb, dU, True)
    dWu = bm.substrate_grad(dH1.to(torch.bfloat16), U.to(torch.bfloat16), alpha)
    dWd = bm.substrate_grad(dZ.to(torch.bfloat16), V.to(torch.bfloat16), alpha)
    dx = torch.zeros_like(x).index_add_(0, tok, dxb)
    torch.cuda.synchronize()

    want = ref.layer_backward_experts(inp, dy64.astype(np.float32).astype(np.float64), R)
    # elementwise: within 3e-5 of |ref| + the expert's (token's) RMS
    for got, ref_, what in ((dthu, want["theta"][0], "theta_up"), (dphu, want["phi"][0], "phi_up"),
                            (dthd, want["theta"][1], "theta_dn"), (dphd, want["phi"][1], "phi_dn")):
        g_ = got.cpu().numpy()
        rms = np.sqrt(np.mean(ref_ ** 2, axis=(1, 2), keepdims=True))
        assert np.all(np.abs(g_ - ref_) <= 3e-5 * (np.abs(ref_) + rms)), f"d{what}"
    dxg = dx.cpu().numpy().astype(np.float64)
    dxw = want["x"]
    assert np.all(np.abs(dxg - dxw) <= 3e-5 * (np.abs(dxw) + np.sqrt(np.mean(dxw ** 2, axis=1, keepdims=True))))
    dg = d_gate.cpu().numpy().reshape(cfg.tokens, k)
    assert np.abs(dg - want["gate"]).max() <= 1e-4 * np.abs(want["gate"]).max()
    # substrate gradients from bf16 copies of both operands: one rounding each
    for got, ref_, mag in ((dWu, want["w_base"][0], want["w_base_abs"][0]),
                           (dWd, want["w_base"][1], want["w_base_abs"][1])):
        assert np.all(np.abs(got.cpu().numpy() - ref_) <= 2.0 ** -7 * mag + 1e-6 * np.abs(ref_).max())
