"""GPU parity: every step of the HIP path against the fp64 oracle.

Per-kernel checks go through the debug hooks of include/bmoe_debug.h; routing
and the whole layer through bmoe_route / bmoe_forward.  Bars:
  * expert indices and bucket layout: bit-exact (tokens the oracle flags as
    within fp64 rounding of a tie may take either choice);
  * layer output: per-token relative L2 error <= 1e-4 (fp32 activations) and
    <= 2e-2 (bf16 activations);
  * integer-valued substrate products: bit-exact after the output rounding.
"""
import math

import numpy as np
import pytest

import compressed_mixture_experts_amd as bm
from compressed_mixture_experts_amd import workloads as wl
from oracle import ref
from gpu_helpers import log, row_rel_err, run_layer, to_dev, to_f64, tol_for

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _cuda():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    bm.lib()
    yield


# ------------------------------------------------------------------ butterfly
@pytest.mark.parametrize("act", ["f32", "bf16"])
@pytest.mark.parametrize("log2n,rows", [(3, 5), (6, 37), (9, 100), (10, 33), (11, 9), (13, 7)])
@pytest.mark.parametrize("transpose", [False, True])
def test_butterfly_kernel(act, log2n, rows, transpose):
    import torch
    n = 1 << log2n
    r = np.random.default_rng(1000 + log2n)
    ang = r.uniform(-math.pi, math.pi, size=(log2n, n // 2)).astype(np.float32)
    x64 = r.standard_normal((rows, n))
    xs = wl.round_to_bf16_bits(x64) if act == "bf16" else x64.astype(np.float32)
    log(f"butterfly act={act} n={n} rows={rows} transpose={transpose}")
    out = bm.dbg_butterfly(torch.from_numpy(ang).cuda(), to_dev(xs, act), transpose=transpose)
    torch.cuda.synchronize()
    got = to_f64(out)
    want = ref.butterfly_apply(ang, ref.stored_to_f64(xs, act).T, transpose=transpose).T
    err = row_rel_err(got, want).max()
    # fp32: a few ulp per stage plus the sin/cos unit; bf16: one output rounding
    assert err <= (2e-5 if act == "f32" else 4e-3), err


@pytest.mark.parametrize("act", ["f32", "bf16"])
def test_butterfly_zero_angles_is_identity_and_inplace(act):
    import torch
    n, rows = 512, 40
    x = wl.round_to_bf16_bits(np.random.default_rng(3).standard_normal((rows, n))) if act == "bf16" \
        else np.random.default_rng(3).standard_normal((rows, n)).astype(np.float32)
    xd = to_dev(x, act)
    x0 = xd.clone()
    ang = torch.zeros((9, n // 2), dtype=torch.float32, device="cuda")
    log(f"butterfly identity act={act}")
    bm.dbg_butterfly(ang, xd, transpose=False, out=xd)  # in place
    torch.cuda.synchronize()
    assert torch.equal(xd, x0)


# ------------------------------------------------------------------ substrate product
@pytest.mark.parametrize("act", ["f32", "bf16"])
@pytest.mark.parametrize("M,N,K", [(1, 64, 64), (37, 128, 512), (300, 192, 256), (515, 512, 2048), (130, 4096, 1024)])
def test_ternary_gemm_integer_exact(act, M, N, K):
    import torch
    r = np.random.default_rng(M + N + K)
    w = r.integers(-1, 2, size=(N, K)).astype(np.int8)
    a = r.integers(-8, 9, size=(M, K)).astype(np.float64)
    a_st = wl.round_to_bf16_bits(a) if act == "bf16" else a.astype(np.float32)
    wp = torch.from_numpy(bm.pack_ternary(w).view(np.int32)).cuda()
    log(f"gemm exact act={act} M={M} N={N} K={K}")
    z = bm.dbg_ternary_gemm(to_dev(a_st, act), wp, N, 1.0)
    torch.cuda.synchronize()
    exact = ref.ternary_product(a, w)           # integers, |.| <= 8 K < 2^24
    want = wl.round_to_bf16_bits(exact) if act == "bf16" else exact.astype(np.float32)
    got = z.cpu().view(torch.int16).numpy().view(np.uint16) if act == "bf16" else z.cpu().numpy()
    assert np.array_equal(got, want)


# ragged last row tiles, one to sixteen column tiles, several K steps, more
# tiles than compute units in the last cases
@pytest.mark.parametrize("M,N,K", [(1, 256, 128), (129, 512, 256), (300, 768, 384), (515, 1024, 2048),
                                   (1000, 4096, 1024), (700, 256, 4096), (4100, 768, 256), (2049, 2048, 640),
                                   (512, 512, 128), (8292, 2048, 256), (20000, 1024, 128)])
def test_ternary_gemm_fp4_integer_exact(M, N, K):
    # integer operands: every partial sum is an exact fp32 integer (|.| <= 8 K < 2^24),
    # so the matrix-core product must round to exactly the bf16 of the true result
    import torch
    r = np.random.default_rng(7 * M + N + K)
    w = r.integers(-1, 2, size=(N, K)).astype(np.int8)
    a = r.integers(-8, 9, size=(M, K)).astype(np.float64)
    a_st = wl.round_to_bf16_bits(a)
    wp = torch.from_numpy(bm.pack_ternary(w).view(np.int32)).cuda()
    log(f"gemm fp4 exact M={M} N={N} K={K}")
    z = bm.dbg_ternary_gemm_fp4(to_dev(a_st, "bf16"), wp, N, 1.0)
    torch.cuda.synchronize()
    want = wl.round_to_bf16_bits(ref.ternary_product(a, w))
    assert np.array_equal(z.cpu().view(torch.int16).numpy().view(np.uint16), want)


@pytest.mark.parametrize("M", [333, 1500])
def test_ternary_gemm_fp4_random_bound(M):
    import torch
    N, K = 512, 1024
    r = np.random.default_rng(10)
    w = r.integers(-1, 2, size=(N, K)).astype(np.int8)
    a_st = wl.round_to_bf16_bits(r.standard_normal((M, K)))
    a = ref.stored_to_f64(a_st, "bf16")
    wp = torch.from_numpy(bm.pack_ternary(w).view(np.int32)).cuda()
    log("gemm fp4 bound")
    z = to_f64(bm.dbg_ternary_gemm_fp4(to_dev(a_st, "bf16"), wp, N, 0.75))
    torch.cuda.synchronize()
    exact = ref.ternary_product(a, w, 0.75)
    # fp32 accumulation of K terms (error <= K u32 sum|a|) plus one bf16 rounding
    bound = K * 2.0 ** -24 * 0.75 * np.abs(a) @ np.abs(w.T).astype(np.float64) + 2.0 ** -8 * np.abs(exact)
    assert np.all(np.abs(z - exact) <= bound + 1e-30)


@pytest.mark.parametrize("act", ["f32", "bf16"])
def test_ternary_gemm_random_bound(act):
    import torch
    M, N, K = 333, 256, 1024
    r = np.random.default_rng(9)
    w = r.integers(-1, 2, size=(N, K)).astype(np.int8)
    a64 = r.standard_normal((M, K))
    a_st = wl.round_to_bf16_bits(a64) if act == "bf16" else a64.astype(np.float32)
    a = ref.stored_to_f64(a_st, act)
    wp = torch.from_numpy(bm.pack_ternary(w).view(np.int32)).cuda()
    log(f"gemm bound act={act}")
    z = to_f64(bm.dbg_ternary_gemm(to_dev(a_st, act), wp, N, 0.75))
    torch.cuda.synchronize()
    exact = ref.ternary_product(a, w, 0.75)
    u = 2.0 ** -23
    gam = K * u / (1 - K * u)
    bound = gam * 0.75 * (np.abs(a) @ np.abs(w.astype(np.float64)).T)
    if act == "bf16":
        bound += np.abs(exact) * 2.0 ** -8   # output rounding to bf16 (one half ulp, doubled)
    assert np.all(np.abs(z - exact) <= bound + 1e-30)


# ------------------------------------------------------------------ routing
def check_routing(inp, idx, gate, offsets=None, slots=None):
    cfg = inp.cfg
    x = ref.stored_to_f64(inp.x, cfg.act)
    wg = ref.stored_to_f64(inp.w_gate, cfg.act)
    R = ref.route(x, wg, cfg.top_k, cfg.renorm_gates)
    idx = np.asarray(idx)
    same = (idx == R.idx).all(axis=1)
    bad = ~same & ~R.ambiguous
    assert not bad.any(), f"{bad.sum()} tokens routed differently, e.g. {np.nonzero(bad)[0][:5]}"
    # gates: fp32 softmax of fp32 logits; relative error bound from the logit bound
    d = cfg.d_model
    depth = d / 32 + 32 if cfg.act == "bf16" else d
    g = depth * 2.0 ** -22
    lerr = 2 * g / (1 - g) * np.linalg.norm(x, axis=1) * np.linalg.norm(wg, axis=1).max()
    tol = (2 * lerr + 3e-5 + cfg.n_experts * 2.0 ** -23)[:, None] * R.gates
    ok = same[:, None]
    assert np.all(~ok | (np.abs(np.asarray(gate, np.float64) - R.gates) <= tol))
    if offsets is not None:
        counts = np.bincount(np.asarray(idx).ravel(), minlength=cfg.n_experts)
        assert np.array_equal(np.asarray(offsets), np.concatenate([[0], np.cumsum(counts)]))
        flat = np.asarray(idx).ravel()
        want = np.concatenate([np.nonzero(flat == e)[0] for e in range(cfg.n_experts)])
        assert np.array_equal(np.asarray(slots), want)
    return R


@pytest.mark.parametrize("ci", [0, 1, 2, 3, 4])
def test_route_configs(ci):
    import torch
    cfg = wl.CONFIGS[ci]
    log(f"route config {cfg.name}")
    inp = wl.generate(cfg)
    layer = bm.Layer.from_inputs(inp)
    idx, gate, off, slots = layer.route(to_dev(inp.x, cfg.act), with_buckets=True)
    torch.cuda.synchronize()
    check_routing(inp, idx.cpu().numpy(), gate.cpu().numpy(), off.cpu().numpy(), slots.cpu().numpy())


def test_route_skewed_and_tied():
    import torch
    cfg = wl.small_config(d_model=128, n_experts=16, top_k=4, tokens=777, act="bf16", seed_index=5)
    inp = wl.generate(cfg, gate_mode="skewed")
    # duplicate two experts' gate rows: exact ties in every token's logits
    inp.w_gate[7] = inp.w_gate[3]
    layer = bm.Layer.from_inputs(inp)
    log("route skewed/tied")
    idx, gate, off, slots = layer.route(to_dev(inp.x, cfg.act), with_buckets=True)
    torch.cuda.synchronize()
    R = check_routing(inp, idx.cpu().numpy(), gate.cpu().numpy(), off.cpu().numpy(), slots.cpu().numpy())
    counts = np.bincount(idx.cpu().numpy().ravel(), minlength=16)
    assert counts.max() > 1.5 * counts.mean()  # the load really is skewed


def test_route_near_ties_top2():
    # near ties resolved exactly: experts 9 and 20 carry expert 5's gate row
    # with one element moved by one bf16 step, and the three rows are three
    # times larger than the rest, so about a quarter of the tokens have two of
    # them on top within the fp32 error bound, their order set by one product.
    # About nine tokens of a 32-token tile are flagged: the first eight are
    # re-ranked from the gate matrix in LDS, the rest through the global path.
    import torch
    cfg = wl.small_config(d_model=512, n_experts=64, top_k=2, tokens=3000, act="bf16", seed_index=9)
    inp = wl.generate(cfg)
    wg = ref.stored_to_f64(inp.w_gate, "bf16")
    inp.w_gate[5] = wl.round_to_bf16_bits(3.0 * wg[5])
    inp.w_gate[9] = inp.w_gate[5]
    inp.w_gate[9, 17] ^= 1
    inp.w_gate[20] = inp.w_gate[5]
    inp.w_gate[20, 300] ^= 1
    layer = bm.Layer.from_inputs(inp)
    log("route near ties, top-2")
    idx, gate, off, slots = layer.route(to_dev(inp.x, cfg.act), with_buckets=True)
    torch.cuda.synchronize()
    R = check_routing(inp, idx.cpu().numpy(), gate.cpu().numpy(), off.cpu().numpy(), slots.cpu().numpy())
    top = np.isin(R.idx, [5, 9, 20]).all(axis=1)
    assert top.mean() > 0.15 and not R.ambiguous[top].any()


def test_route_buckets_beyond_one_round():
    # more routed slots than one bucketing round (65536): bucket bases must
    # count the slots of lower experts in every round
    import torch
    cfg = wl.small_config(d_model=64, n_experts=8, top_k=2, tokens=40000, act="bf16", seed_index=6)
    inp = wl.generate(cfg, gate_mode="skewed")
    layer = bm.Layer.from_inputs(inp)
    log("route 80000 slots")
    idx, gate, off, slots = layer.route(to_dev(inp.x, cfg.act), with_buckets=True)
    torch.cuda.synchronize()
    check_routing(inp, idx.cpu().numpy(), gate.cpu().numpy(), off.cpu().numpy(), slots.cpu().numpy())


def test_route_wide_tokens_128_token_tiles():
    # bf16 tokens too wide for the whole-tile router and at least 32768 of
    # them: 128-token tiles of eight waves.  A ragged last tile, 100 experts
    # (a partial last block of 16) and k = 3 (the decision over the logits in
    # LDS); the gate matrix read from the prepared fragment copy and from W_g.
    import torch
    cfg = wl.small_config(d_model=1024, n_experts=100, top_k=3, tokens=32768 + 77, act="bf16", seed_index=13)
    inp = wl.generate(cfg)
    for prepared in (True, False):
        layer = bm.Layer.from_inputs(inp)
        if prepared:
            layer.prepare()
        log(f"route 128-token tiles, prepared={prepared}")
        idx, gate, off, slots = layer.route(to_dev(inp.x, cfg.act), with_buckets=True)
        torch.cuda.synchronize()
        check_routing(inp, idx.cpu().numpy(), gate.cpu().numpy(), off.cpu().numpy(), slots.cpu().numpy())


# ------------------------------------------------------------------ layer forward
def check_forward(inp, y, idx, gate, tokens=None):
    """Compare the GPU layer output with the oracle on every token (the
    materialised definition) or on the given tokens (the oracle's right-to-left
    products, stacked per expert).  Routing is compared on every token; tokens
    the oracle flags as within fp64 rounding of a tie are evaluated at the
    GPU's choice."""
    cfg = inp.cfg
    y = to_f64(y)
    idx = idx.cpu().numpy()
    x = ref.stored_to_f64(inp.x, cfg.act)
    wg = ref.stored_to_f64(inp.w_gate, cfg.act)
    R = ref.route(x, wg, cfg.top_k, cfg.renorm_gates)
    mism = ~(idx == R.idx).all(axis=1)
    assert not (mism & ~R.ambiguous).any()
    if tokens is None:
        yref, _ = ref.forward(inp, routing=R, idx_override=idx if mism.any() else None)
        err = row_rel_err(y, yref)
    else:
        tokens = np.asarray(tokens)
        yref, _, _ = ref.forward_tokens(inp, tokens, routing=R,
                                        idx_override=idx[tokens] if mism[tokens].any() else None)
        err = row_rel_err(y[tokens], yref)
    log(f"  {len(err)} tokens: max rel err {err.max():.3e} p99 {np.quantile(err, 0.99):.3e} "
        f"mean {err.mean():.3e} (bar {tol_for(cfg.act):.0e})")
    assert err.max() <= tol_for(cfg.act), err.max()
    return err


@pytest.mark.parametrize("ci", [0, 1, 2])
def test_forward_configs_full(ci):
    cfg = wl.CONFIGS[ci]
    log(f"forward config {cfg.name}")
    inp = wl.generate(cfg)
    _, _, (y, idx, gate) = run_layer(inp)
    check_forward(inp, y, idx, gate)


def test_forward_vit_ffn_every_token():
    # the ViT-style FFN layer (8192 tokens): every token against the oracle's
    # right-to-left products
    cfg = wl.CONFIGS[3]
    log(f"forward config {cfg.name}, every token")
    inp = wl.generate(cfg)
    _, _, (y, idx, gate) = run_layer(inp)
    check_forward(inp, y, idx, gate, tokens=np.arange(cfg.tokens))


def bucket_edge_tokens(off, slots, k, tile=64, per_expert_tiles=2):
    """Tokens whose rows sit at the edges of the expert tiles: for every expert
    with rows, its first and last bucket rows and the first and last row of
    its first `per_expert_tiles` tiles of `tile` rows."""
    off = np.asarray(off)
    slots = np.asarray(slots)
    pos = []
    for e in range(len(off) - 1):
        a, b = int(off[e]), int(off[e + 1])
        if b <= a:
            continue
        pos += [a, b - 1]
        for j in range(per_expert_tiles):
            for q in (a + j * tile, a + (j + 1) * tile - 1):
                if a <= q < b:
                    pos.append(q)
    return np.unique(slots[np.asarray(pos)] // k)


def test_forward_large_every_expert():
    # the large FFN layer with outliers (32768 tokens, 256 experts): at least
    # one token of every expert, the first and last rows of the first two
    # 64-row tiles of every expert, and a seeded random sample
    import torch
    cfg = wl.CONFIGS[4]
    log(f"forward config {cfg.name}, tile-edge tokens of every expert")
    inp = wl.generate(cfg)
    layer, x, (y, idx, gate) = run_layer(inp)
    _, _, off, slots = layer.route(x, with_buckets=True)
    torch.cuda.synchronize()
    off, slots = off.cpu().numpy(), slots.cpu().numpy()
    toks = bucket_edge_tokens(off, slots, cfg.top_k)
    r = np.random.default_rng(4)
    toks = np.unique(np.concatenate([toks, r.choice(cfg.tokens, size=64, replace=False),
                                     [0, cfg.tokens - 1]]))
    chosen = np.unique(idx.cpu().numpy()[toks])
    log(f"  {len(toks)} tokens covering {len(chosen)} of {cfg.n_experts} experts")
    assert len(chosen) == int((np.diff(off) > 0).sum())
    check_forward(inp, y, idx, gate, tokens=toks)
    assert bool(torch.isfinite(y.float()).all())


SMALL_CASES = [
    dict(d_model=64, n_experts=5, top_k=2, tokens=37, act="bf16"),
    dict(d_model=64, n_experts=5, top_k=2, tokens=37, act="f32"),
    dict(d_model=128, n_experts=1, top_k=1, tokens=1, act="bf16"),
    dict(d_model=256, n_experts=8, top_k=8, tokens=300, act="bf16"),
    dict(d_model=64, n_experts=3, top_k=1, tokens=129, act="bf16"),
    dict(d_model=128, n_experts=6, top_k=3, tokens=200, act="f32", renorm_gates=True, w_scale=0.5),
    dict(d_model=64, d_ff=256, n_experts=3, top_k=2, tokens=50, act="bf16"),
    dict(d_model=64, d_ff=128, n_experts=4, top_k=2, tokens=65, act="f32"),
    dict(d_model=128, d_ff=64, n_experts=7, top_k=2, tokens=333, act="bf16", renorm_gates=True),
    dict(d_model=256, d_ff=1024, n_experts=16, top_k=2, tokens=1000, act="bf16", ffn_act="none"),
    # wide bf16 rows: butterflies as low / high parts, several 64-row blocks per expert
    dict(d_model=1024, n_experts=6, top_k=2, tokens=400, act="bf16"),
    dict(d_model=2048, n_experts=3, top_k=1, tokens=50, act="bf16"),
    dict(d_model=256, d_ff=4096, n_experts=5, top_k=2, tokens=120, act="bf16"),
    dict(d_model=128, d_ff=8192, n_experts=3, top_k=2, tokens=40, act="bf16"),
    # width 8192 with the up product's epilogue: several 128-row product tiles
    # spanning two experts, 64-row middle tiles with ragged tails
    dict(d_model=256, d_ff=8192, n_experts=5, top_k=2, tokens=301, act="bf16"),
    dict(d_model=256, d_ff=8192, n_experts=1, top_k=1, tokens=1, act="bf16"),
    # top-1: the output rotation's high part writes y directly; one token
    dict(d_model=1024, d_ff=4096, n_experts=4, top_k=1, tokens=100, act="bf16"),
    dict(d_model=2048, d_ff=1024, n_experts=8, top_k=2, tokens=1, act="bf16"),
    # d_ff 4096: the up product's epilogue applies phi_up's low part; 64 experts
    # with about 3 rows each, so most 16-row blocks hold several experts, and a
    # ragged last row tile
    dict(d_model=256, d_ff=4096, n_experts=64, top_k=2, tokens=101, act="bf16"),
    # the same with a few long experts (row tiles inside one expert) and k = 1
    dict(d_model=256, d_ff=4096, n_experts=3, top_k=1, tokens=700, act="bf16"),
]


@pytest.mark.parametrize("case", range(len(SMALL_CASES)))
def test_forward_small(case):
    kw = SMALL_CASES[case]
    cfg = wl.small_config(seed_index=200 + case, **kw)
    log(f"forward small {cfg.name} {kw}")
    inp = wl.generate(cfg)
    _, _, (y, idx, gate) = run_layer(inp)
    check_forward(inp, y, idx, gate)


def test_forward_identity_experts_and_skew():
    cfg = wl.small_config(d_model=512, n_experts=32, top_k=2, tokens=2048, act="bf16", seed_index=77)
    inp = wl.generate(cfg, angle_mode="zero", gate_mode="skewed")
    log("forward identity experts, skewed routing")
    _, _, (y, idx, gate) = run_layer(inp)
    check_forward(inp, y, idx, gate)


def test_forward_ffn_skewed_routing():
    # skewed gates at FFN widths: some experts get no rows, others several
    # 64-row tiles of the split butterflies
    cfg = wl.small_config(d_model=1024, d_ff=4096, n_experts=16, top_k=2, tokens=600, act="bf16",
                          seed_index=78)
    inp = wl.generate(cfg, gate_mode="skewed")
    log("forward FFN skewed routing")
    _, _, (y, idx, gate) = run_layer(inp)
    counts = np.bincount(idx.cpu().numpy().ravel(), minlength=16)
    assert counts.max() > 64 and counts.min() < counts.mean() / 2
    check_forward(inp, y, idx, gate)


def test_forward_outliers_small():
    cfg = wl.small_config(d_model=256, d_ff=512, n_experts=8, top_k=2, tokens=300, act="bf16",
                          outlier_frac=0.02, outlier_scale=50.0, seed_index=31)
    inp = wl.generate(cfg)
    log("forward outliers small")
    _, _, (y, idx, gate) = run_layer(inp)
    check_forward(inp, y, idx, gate)


def test_forward_deterministic_and_empty():
    import torch
    cfg = wl.CONFIGS[1]
    inp = wl.generate(cfg)
    layer = bm.Layer.from_inputs(inp)
    x = to_dev(inp.x, cfg.act)
    log("forward determinism")
    y1 = layer.forward(x)
    y2 = layer.forward(x)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)
    y0 = layer.forward(x[:0])
    torch.cuda.synchronize()
    assert y0.shape == (0, cfg.d_model)


def test_forward_tile_heights_agree():
    # width-512 square layers run 32-row expert tiles when those would fill two
    # per CU, else 48-row tiles when those fit one per CU, else 64-row tiles;
    # every row gets the same arithmetic whatever the height.  On 256 CUs the
    # 4096 tokens take 48-row tiles, 5000 tokens 64-row tiles and 16384 tokens
    # 32-row tiles: the outputs of shared tokens must agree bit for bit
    # (routing is per token, so it is the same).
    import torch
    cfg = wl.CONFIGS[1]
    inp = wl.generate(cfg)
    layer = bm.Layer.from_inputs(inp)
    x = to_dev(inp.x, cfg.act)
    n = x.shape[0]
    log("forward tile heights 48 / 64 / 32")
    y1 = layer.forward(x)
    y5 = layer.forward(torch.cat([x, x[:904]]).contiguous())
    y4 = layer.forward(torch.cat([x, x, x, x]).contiguous())
    torch.cuda.synchronize()
    assert torch.equal(y1, y5[:n])
    assert torch.equal(y1, y4[:n])
    assert torch.equal(y4[:n], y4[3 * n:])


def test_route_matches_forward_routing():
    import torch
    cfg = wl.CONFIGS[2]
    inp = wl.generate(cfg)
    layer = bm.Layer.from_inputs(inp)
    x = to_dev(inp.x, cfg.act)
    log("route vs forward routing")
    i1, g1 = layer.route(x)
    _, i2, g2 = layer.forward(x, return_routing=True)
    torch.cuda.synchronize()
    assert torch.equal(i1, i2) and torch.equal(g1, g2)


# Prepared weights (bmoe_prepare, done once per weight set) must give exactly the
# results of the per-call preparation: same kernels on the same bytes.
PREP_CASES = [
    dict(d_model=512, n_experts=64, top_k=2, tokens=700),   # matrix-core expert kernel
    dict(d_model=256, d_ff=1024, n_experts=6, top_k=2, tokens=300),   # fp4 substrates of both GEMMs
    dict(d_model=128, d_ff=4096, n_experts=4, top_k=2, tokens=150),   # + low-part block factors
    dict(d_model=1024, n_experts=5, top_k=2, tokens=200),   # square width 1024: low and high factors
    dict(d_model=256, n_experts=9, top_k=3, tokens=333),
    dict(d_model=128, n_experts=5, top_k=2, tokens=200),    # fp32-rotation expert kernel
    dict(d_model=64, n_experts=3, top_k=1, tokens=65),
]


@pytest.mark.parametrize("case", range(len(PREP_CASES)))
def test_prepared_matches_per_call(case):
    import torch
    kw = PREP_CASES[case]
    cfg = wl.small_config(seed_index=400 + case, act="bf16", **kw)
    log(f"prepared vs per call {cfg.name}")
    inp = wl.generate(cfg)
    layer = bm.Layer.from_inputs(inp, device="cuda")
    x = to_dev(inp.x, cfg.act)
    assert "prep" in layer.kernel_names()
    y0, i0, g0 = layer.forward(x, return_routing=True)
    layer.prepare()
    assert layer.struct.prepared and layer.prepared_bytes() > 0
    assert "prep" not in layer.kernel_names()
    y1, i1, g1 = layer.forward(x, return_routing=True)
    torch.cuda.synchronize()
    assert torch.equal(i0, i1) and torch.equal(g0, g1)
    assert torch.equal(y0.view(torch.int16), y1.view(torch.int16))
    check_forward(inp, y1, i1, g1)


@pytest.mark.parametrize("ci", [1, 2])
def test_forward_configs_prepared(ci):
    cfg = wl.CONFIGS[ci]
    log(f"forward config {cfg.name} with prepared weights")
    inp = wl.generate(cfg)
    _, _, (y, idx, gate) = run_layer(inp, prepared=True)
    check_forward(inp, y, idx, gate)


@pytest.mark.parametrize("ci", [1, 3])
def test_graph_replay_matches_eager(ci):
    # a captured HIP graph of one forward, replayed several times with eager
    # forwards and synchronisations in between, reproduces the eager result
    import torch
    cfg = wl.CONFIGS[ci]
    inp = wl.generate(cfg)
    layer = bm.Layer.from_inputs(inp, device="cuda")
    layer.prepare()
    x = to_dev(inp.x, cfg.act)
    log(f"graph replay {cfg.name}")
    y_eager = layer.forward(x).clone()
    y = torch.empty_like(x)
    layer.forward(x, y)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=torch.cuda.Stream()):
        layer.forward(x, y)
    for rep in range(3):
        y.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), y_eager.view(torch.int16)), rep
        y_other = layer.forward(x)          # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(y_other.view(torch.int16), y_eager.view(torch.int16))
