#!/usr/bin/env python3
"""Routed tokens/s of one ButterflyMoE layer forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config I]

One step = one bmoe_forward over a batch of synthetic tokens (router,
bucketing, input rotation, ternary substrate product(s), FFN middle when
present, output rotation and combine), inputs resident in HBM.  Prints one
JSON line.  The dominant kernel's duration is measured live with HIP events
recorded around that kernel's launch inside the timed steps; the CPU baseline
is the fp64 oracle timed on this host over a bounded sample of the same
workload.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0  # dense bf16 MFMA
VALU_FP32_PEAK_TFLOPS = 157.3


class HipEvents:
    """Raw hipEvent_t handles through the HIP runtime (timing plumbing only)."""

    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self, n):
        out = []
        for _ in range(n):
            e = ctypes.c_void_p()
            rc = self.hip.hipEventCreate(ctypes.byref(e))
            if rc != 0:
                raise RuntimeError(f"hipEventCreate failed ({rc})")
            out.append(e.value)
        return out

    def elapsed_ms(self, a, b):
        ms = ctypes.c_float(0.0)
        rc = self.hip.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(a), ctypes.c_void_p(b))
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return float(ms.value)

    def destroy(self, evs):
        for e in evs:
            self.hip.hipEventDestroy(ctypes.c_void_p(e))


def kernel_work(cfg):
    """Algorithmic bytes and flops of each kernel of one forward.

    Bytes count what the step must move at least once (activations in and out
    of each kernel, the packed substrate, the angles of every expert, the
    router weights); flops count multiply-adds as 2.  Returns
    {name: (bytes, flops, bound)}."""
    s = 2 if cfg.act == "bf16" else 4
    T, d, f, N, k = cfg.tokens, cfg.d_model, cfg.d_ff, cfg.n_experts, cfg.top_k
    R = T * k
    Ld = int(math.log2(d))
    ang_d = N * Ld * (d // 2) * 4
    w = {}
    # the router also leaves each token tile's slots ordered by expert (R
    # indices) and the first position of every expert in each tile's list
    bt = 64 if T >= 64 * 256 else 32 if T >= 32 * 256 else 16
    G = (T + bt - 1) // bt
    w["route"] = (T * d * s + N * d * s + 8 * R + 4 * R + 4 * G * N, 2 * T * d * N, "hbm")
    w["bucket"] = (4 * R + 4 * G * N + 4 * R + 4 * (N + 1), 0, "hbm")

    def split(L):
        # bf16 rows of width 1024 .. 8192: butterflies as low / high parts
        return cfg.act == "bf16" and 10 <= L <= 13

    def part(n, stages, nbfly=1, extra=0):
        # one pass over R rows of width n applying `stages` stages of nbfly butterflies
        return (2 * R * n * s + nbfly * N * stages * (n // 2) * 4 + extra,
                6 * R * (n // 2) * stages * nbfly, "hbm")

    def lowfac_bytes(L):
        # low-part block factors per expert (widths 1024 .. 8192, bf16 layers)
        if cfg.act != "bf16" or not 10 <= L <= 13:
            return 0
        w = 1 << L
        return 16 * ((w // 16) * max(16, w // 256) * 2 + (w // 256) * 512)

    def highfac_bytes(L):
        # high-part block factors per expert (one 16 x 16 bf16 block per column)
        return (1 << (L - 4)) * 512 if cfg.act == "bf16" and 10 <= L <= 13 else 0

    def high(n, nbfly=1, extra=0):
        L = int(math.log2(n))
        return (2 * R * n * s + nbfly * N * highfac_bytes(L) + extra, 2 * R * n * 16 * nbfly, "hbm")

    def low(n):
        # low part of width n: block factors on the matrix cores where prepared
        L = int(math.log2(n))
        fb = lowfac_bytes(L)
        if not fb:
            return part(n, L - 4)
        B0 = max(16, 1 << (L - 8))
        return (2 * R * n * s + N * fb, 2 * R * n * (B0 + 16), "hbm")

    prep_lo = prep_hi = 0

    if split(Ld):
        w["bfly_in_hi"] = high(d, extra=4 * R)
        w["bfly_in_lo"] = low(d)
        prep_lo += N * (Ld * (d // 2) * 4 + lowfac_bytes(Ld)) if lowfac_bytes(Ld) else 0
        prep_hi += 2 * N * (4 * (d // 2) * 4 + highfac_bytes(Ld))
    else:
        w["bfly_in"] = (2 * R * d * s + ang_d + 4 * R, 6 * R * (d // 2) * Ld, "hbm")

    def fp4_gemm(din, dout):
        # bf16 products whose shape the fp4 matrix-core GEMM covers read the
        # substrate prepared as fp4 (half a byte per weight)
        return cfg.act == "bf16" and dout % 256 == 0 and din % 128 == 0

    def gemm(din, dout):
        fl = 2 * R * din * dout
        by = R * din * s + R * dout * s + dout * din // (2 if fp4_gemm(din, dout) else 4)
        return (by, fl, "mfma" if fl / by > MFMA_BF16_PEAK_TFLOPS / HBM_PEAK_GBS * 1e3 else "hbm")

    if f == 0:
        w["gemm"] = gemm(d, d)
        if fp4_gemm(d, d) and Ld > 9:
            w["prep"] = (d * d // 4 + d * d // 2, 0, "hbm")
        if cfg.act == "bf16" and Ld in (8, 9):
            # rotations as block factors on the matrix cores: per rotation one
            # P x P and one 16 x 16 product per 32-wide / 16-wide block of a row
            P = 32 if Ld == 9 else 16
            fac = N * 2 * (P * 64 * 4 * 2 + 16 * (P // 16) * 64 * (P // 4) * 2)
            w["prep"] = (d * d // 4 + d * d // 2 + 2 * ang_d + fac, 0, "hbm")
            fb = 2 * R * d * s + fac + d * d // 2 + 8 * R
            ff = 2 * R * d * d + 2 * 2 * R * d * (P + 16)
        else:
            fb = 2 * R * d * s + 2 * ang_d + d * d // 4 + 8 * R
            ff = 2 * R * d * d + 2 * 6 * R * (d // 2) * Ld
            w["prep"] = (d * d // 4 + d * d, 0, "hbm")
        w["fused"] = (fb, ff, "mfma" if ff / fb > MFMA_BF16_PEAK_TFLOPS / HBM_PEAK_GBS * 1e3 else "hbm")
    else:
        Lf = int(math.log2(f))
        w["gemm_up"] = gemm(d, f)
        if split(Lf):
            w["bfly_mid_lo"] = low(f)
            w["bfly_mid_hi"] = high(f, nbfly=2)
            w["bfly_mid_lo_t"] = low(f)
            prep_lo += 2 * N * (Lf * (f // 2) * 4 + lowfac_bytes(Lf)) if lowfac_bytes(Lf) else 0
            prep_hi += 2 * N * (4 * (f // 2) * 4 + highfac_bytes(Lf))
        else:
            w["bfly_mid"] = (2 * R * f * s + 2 * N * Lf * (f // 2) * 4, 2 * 6 * R * (f // 2) * Lf, "hbm")
        w["gemm_down"] = gemm(f, d)
        pw = sum(a * b // 4 + a * b // 2 for a, b in ((d, f), (f, d)) if fp4_gemm(a, b))
        if pw:
            w["prep"] = (pw, 0, "hbm")
    if split(Ld):
        w["bfly_out_lo"] = low(d)
        prep_lo += N * (Ld * (d // 2) * 4 + lowfac_bytes(Ld)) if lowfac_bytes(Ld) else 0
        w["bfly_out_hi"] = high(d, extra=8 * R)
    else:
        w["bfly_out"] = (2 * R * d * s + ang_d + 8 * R, 6 * R * (d // 2) * Ld, "hbm")
    if prep_lo:
        w["prep_lo"] = (prep_lo, 0, "hbm")
    if prep_hi:
        w["prep_hi"] = (prep_hi, 0, "hbm")
    if k > 1:
        w["combine"] = (R * d * s + T * d * s, R * d, "hbm")
    return w


def roofline_entry(by, fl, bound, seconds, traffic=None):
    if bound == "mfma":
        ach = fl / seconds / 1e12
        return {"bound": "mfma", "achieved": round(ach, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(ach / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": traffic}
    ach = by / seconds / 1e9
    return {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": traffic}


def cpu_baseline(inp, y_gpu, seconds_target: float):
    """fp64 oracle on this host: full-batch forwards until ~seconds_target."""
    import numpy as np
    from oracle import ref
    try:
        from threadpoolctl import threadpool_info
        cores = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        cores = os.cpu_count() or 1
    cfg = inp.cfg
    t0 = time.perf_counter()
    reps = 0
    y_ref = None
    while True:
        y_ref, _ = ref.forward(inp)
        reps += 1
        if time.perf_counter() - t0 >= seconds_target:
            break
    dt = time.perf_counter() - t0
    err = None
    if y_gpu is not None:
        num = np.linalg.norm(y_gpu - y_ref, axis=1)
        den = np.maximum(np.linalg.norm(y_ref, axis=1), 1e-30)
        err = float((num / den).max())
    return {"value": round(cfg.tokens * reps / dt, 1), "unit": "tokens/s", "cores": int(cores),
            "kind": "oracle",
            "sample": f"{reps} full-batch forward(s) of {cfg.tokens} tokens ({cfg.name}), "
                      f"materialising every used expert in fp64, {dt:.1f} s",
            "max_rel_err_gpu_vs_oracle": err}


def spread_stats(v):
    """Per-row outlier statistics of v [rows][n] (float32 tensor), averaged over rows:
    peak-to-RMS ratio max|v| / rms(v), and the relative squared error of the
    ternary code {-a, 0, +a} of each row (threshold 0.7 mean|v|, a = mean of
    the |v| above it), |v - q|^2 / |v|^2."""
    import torch
    a = v.abs()
    rms = v.pow(2).mean(1).sqrt()
    peak = a.max(1).values / rms
    m = a > 0.7 * a.mean(1, keepdim=True)
    alpha = (a * m).sum(1, keepdim=True) / m.sum(1, keepdim=True).clamp(min=1)
    q = alpha * torch.sign(v) * m
    err = (v - q).pow(2).sum(1) / v.pow(2).sum(1)
    return float(peak.mean()), float(err.mean())


def outlier_spread(n_experts: int = 8) -> dict:
    """Large FFN workload's tokens (1% of channels x50) before and after the
    input rotation B(theta_e)^T of the up substrate, random angles, for the
    first n_experts experts: mean peak-to-RMS ratio, ternary-code error and
    the share of the energy in the outlier channels."""
    import numpy as np
    import torch
    import compressed_mixture_experts_amd as bm
    from compressed_mixture_experts_amd import workloads as wl
    cfg = wl.CONFIGS[4]
    inp = wl.generate(cfg)
    xb = torch.from_numpy(inp.x.view(np.int16)).view(torch.bfloat16).cuda()
    x = xb.float()
    ch = torch.from_numpy(np.asarray(inp.outlier_channels)).cuda()

    def share(v):
        e = v.pow(2)
        return float((e[:, ch].sum(1) / e.sum(1)).mean())

    p0, q0 = spread_stats(x)
    rot = []
    for e in range(n_experts):
        th = torch.from_numpy(np.ascontiguousarray(inp.theta[0][e], dtype=np.float32)).cuda()
        u = bm.dbg_butterfly(th, x, transpose=True)
        rot.append((*spread_stats(u), share(u)))
    torch.cuda.synchronize()
    r = np.array(rot)
    return {"measurement": "outlier spread by the input rotation (random angles)",
            "workload": cfg.name, "tokens": cfg.tokens, "width": cfg.d_model,
            "outlier_channels": int(len(ch)), "experts": n_experts,
            "x": {"peak_to_rms": round(p0, 3), "ternary_rel_err": round(q0, 4), "outlier_energy_share": round(share(x), 4)},
            "rotated": {"peak_to_rms": round(float(r[:, 0].mean()), 3), "ternary_rel_err": round(float(r[:, 1].mean()), 4),
                        "outlier_energy_share": round(float(r[:, 2].mean()), 4)}}


def grad_measure(reps: int = 20) -> dict:
    """Butterfly backward (bmoe_butterfly_backward) at the routed-row shapes of
    the edge workload (input rotation, width 512), the ViT FFN workload (input
    rotation, width 1024) and the large workload
    (input rotation, width 2048; FFN up rotation, width 8192): bf16 rows
    bucketed evenly over the experts, fp32 angles.  Per shape: mean time per
    call (HIP events on torch's stream) and the rate of its algorithmic HBM
    bytes (rows x, dy in and dx out, angles in, angle gradients out; per-chunk
    partial gradients and, at widths of 4096 and more, the fp32 rows between the
    part passes are the implementation's own traffic and not counted)."""
    import math
    import torch
    import compressed_mixture_experts_amd as bm
    out = []
    for name, rows, n, N, tr in (("edge_d512_n64 input rotation", 8192, 512, 64, True),
                                 ("vit_ffn_d1024_n64 input rotation", 16384, 1024, 64, True),
                                 ("large_d2048_n256 input rotation", 65536, 2048, 256, True),
                                 ("large_d2048_n256 ffn up rotation", 65536, 8192, 256, False)):
        L = int(math.log2(n))
        g = torch.Generator(device="cuda").manual_seed(11)
        x = torch.randn((rows, n), device="cuda", generator=g).to(torch.bfloat16)
        dy = torch.randn((rows, n), device="cuda", generator=g).to(torch.bfloat16)
        ang = (torch.rand((N, L, n // 2), device="cuda", generator=g) * 2 - 1) * math.pi
        off = torch.tensor([(rows * e) // N for e in range(N + 1)], dtype=torch.int32, device="cuda")
        dx = torch.empty_like(x)
        for _ in range(3):
            bm.butterfly_backward(ang, off, x, dy, tr, dx=dx)
        s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        s0.record()
        for _ in range(reps):
            bm.butterfly_backward(ang, off, x, dy, tr, dx=dx)
        s1.record()
        torch.cuda.synchronize()
        ms = s0.elapsed_time(s1) / reps
        by = 3 * rows * n * 2 + 2 * N * L * (n // 2) * 4
        out.append({"shape": name, "rows": rows, "width": n, "experts": N, "ms": round(ms, 4),
                    "hbm_gbps": round(by / (ms * 1e-3) / 1e9, 1), "hbm_frac": round(by / (ms * 1e-3) / 8e12, 4)})
    # the substrate's latent gradient (straight-through): dW = alpha dZ^T U over
    # all routed rows; flops 2 rows d_out d_in against the bf16 MFMA peak
    sg = []
    for name, rows, d_out, d_in in (("edge_d512_n64 substrate", 16384, 512, 512),
                                    ("large_d2048_n256 ffn up substrate", 65536, 8192, 2048),
                                    ("large_d2048_n256 ffn down substrate", 65536, 2048, 8192)):
        g = torch.Generator(device="cuda").manual_seed(12)
        dz = torch.randn((rows, d_out), device="cuda", generator=g).to(torch.bfloat16)
        u = torch.randn((rows, d_in), device="cuda", generator=g).to(torch.bfloat16)
        dw = torch.empty((d_out, d_in), device="cuda")
        for _ in range(3):
            bm.substrate_grad(dz, u, 1.0, dw=dw)
        s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        s0.record()
        for _ in range(reps):
            bm.substrate_grad(dz, u, 1.0, dw=dw)
        s1.record()
        torch.cuda.synchronize()
        ms = s0.elapsed_time(s1) / reps
        tf = 2.0 * rows * d_out * d_in / (ms * 1e-3) / 1e12
        sg.append({"shape": name, "rows": rows, "d_out": d_out, "d_in": d_in, "ms": round(ms, 4),
                   "tflops": round(tf, 1), "mfma_frac": round(tf / 2500.0, 4)})
        del dz, u, dw
    # the gated combine's backward at the edge and large routed-row shapes:
    # bytes dy rows gathered, expert outputs and row gradients, gates in and out
    cb = []
    for name, T, d in (("edge_d512_n64 combine", 4096, 512), ("large_d2048_n256 combine", 32768, 2048)):
        k = 2
        g = torch.Generator(device="cuda").manual_seed(13)
        dy = torch.randn((T, d), device="cuda", generator=g).to(torch.bfloat16)
        o = torch.randn((T * k, d), device="cuda", generator=g).to(torch.bfloat16)
        slots = torch.randperm(T * k, device="cuda", generator=g).to(torch.int32)
        gate = torch.rand(T * k, device="cuda", generator=g)
        for _ in range(3):
            bm.combine_backward(dy, slots, gate, k, o)
        s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        s0.record()
        for _ in range(reps):
            bm.combine_backward(dy, slots, gate, k, o)
        s1.record()
        torch.cuda.synchronize()
        ms = s0.elapsed_time(s1) / reps
        by = 3 * T * k * d * 2 + T * k * 16
        cb.append({"shape": name, "rows": T * k, "width": d, "ms": round(ms, 4),
                   "hbm_gbps": round(by / (ms * 1e-3) / 1e9, 1), "hbm_frac": round(by / (ms * 1e-3) / 8e12, 4)})
        del dy, o
    # the router's backward (softmax at the chosen experts -> logits -> W_g, x):
    # flops 2 T d N for each of the logits, dx and dW_g
    rb = []
    for name, T, d, N in (("edge_d512_n64 router", 4096, 512, 64), ("large_d2048_n256 router", 32768, 2048, 256)):
        g = torch.Generator(device="cuda").manual_seed(14)
        x = torch.randn((T, d), device="cuda", generator=g).to(torch.bfloat16)
        wg = (torch.randn((N, d), device="cuda", generator=g) / math.sqrt(d)).to(torch.bfloat16)
        idx = torch.argsort(torch.rand((T, N), device="cuda", generator=g), dim=1)[:, :2].to(torch.int32).contiguous()
        dg = torch.randn((T, 2), device="cuda", generator=g)
        for _ in range(3):
            bm.router_backward(x, wg, idx, dg)
        s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        s0.record()
        for _ in range(reps):
            bm.router_backward(x, wg, idx, dg)
        s1.record()
        torch.cuda.synchronize()
        ms = s0.elapsed_time(s1) / reps
        rb.append({"shape": name, "tokens": T, "width": d, "experts": N, "ms": round(ms, 4),
                   "tflops": round(3 * 2.0 * T * d * N / (ms * 1e-3) / 1e12, 2)})
        del x, wg, idx
    return {"measurement": "layer backward pieces: butterfly backward; substrate weight gradient; combine backward; "
                           "router backward",
            "dtype": "bf16 rows, fp32 angles and weight gradients", "shapes": out, "substrate": sg, "combine": cb,
            "router": rb}


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", type=int, default=None,
                    help="workload index (default: the d=512, 64-expert layer)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="only copy a MIB-MiB device buffer 5 times (HBM counter calibration) and exit")
    ap.add_argument("--per-call-prep", action="store_true",
                    help="re-encode the weights inside every forward instead of once")
    ap.add_argument("--eager", action="store_true",
                    help="time launch-by-launch forwards instead of captured-graph replays")
    ap.add_argument("--grad", action="store_true",
                    help="only time the butterfly backward at the workloads' routed-row shapes and exit")
    ap.add_argument("--outlier-spread", action="store_true",
                    help="only measure how the input rotation spreads the large workload's "
                         "activation outliers (peak-to-RMS ratio, ternary-code error) and exit")
    ap.add_argument("--skewed", action="store_true",
                    help="skewed routing: gate row e scaled by 4/(e+1)^0.75, so a few experts take "
                         "most of the rows and many get few or none")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU (asked for --gpus {args.gpus}): the ButterflyMoE forward "
              "shards over tokens with no exchange between GPUs, so N GPUs would each run this "
              "same step on their own T/N tokens.", file=sys.stderr)
        return 2

    import numpy as np
    import torch
    if args.copy_probe:
        src = torch.empty(args.copy_probe << 20, dtype=torch.uint8, device="cuda")
        src.fill_(1)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_mib": args.copy_probe, "copies": 5}))
        return 0
    if args.outlier_spread:
        print(json.dumps(outlier_spread()))
        return 0
    if args.grad:
        print(json.dumps(grad_measure()))
        return 0
    import compressed_mixture_experts_amd as bm
    from compressed_mixture_experts_amd import workloads as wl

    ci = wl.BENCH_CONFIG_INDEX if args.config is None else args.config
    cfg = wl.CONFIGS[ci]
    wname = cfg.name + ("_skewed" if args.skewed else "")
    print(f"[bench] workload {wname}: generating inputs", file=sys.stderr, flush=True)
    inp = wl.generate(cfg, gate_mode="skewed" if args.skewed else "normal")
    layer = bm.Layer.from_inputs(inp, device="cuda")
    # weight preparation (substrate re-encoding, rotation block factors): once per
    # weight set, outside the timed steps, unless --per-call-prep
    prep_ms = None
    if not args.per_call_prep and layer.prepared_bytes() > 0:
        layer.prepare()
        torch.cuda.synchronize()
        t_p = time.perf_counter()
        layer.prepare()
        torch.cuda.synchronize()
        prep_ms = (time.perf_counter() - t_p) * 1e3
    if cfg.act == "bf16":
        x = torch.from_numpy(inp.x.view(np.int16)).view(torch.bfloat16).cuda()
    else:
        x = torch.from_numpy(inp.x).cuda()
    y = torch.empty_like(x)
    # rows per expert of this batch's routing (load balance of the workload)
    idx = layer.route(x)[0]
    counts = torch.bincount(idx.reshape(-1).long(), minlength=cfg.n_experts).cpu().numpy()
    load = {"rows_max_expert": int(counts.max()), "rows_mean_expert": round(float(counts.mean()), 1),
            "experts_without_rows": int((counts == 0).sum())}
    names = layer.kernel_names()
    nk = len(names)
    ev = HipEvents()

    print(f"[bench] warmup {args.warmup} steps", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        layer.forward(x, y)
    torch.cuda.synchronize()

    # calibration (outside the timed region): every kernel bracketed
    cal_steps = 10
    marks = [ev.create(nk + 1) for _ in range(cal_steps)]
    for i in range(cal_steps):
        layer.forward_marked(x, y, marks[i])
    torch.cuda.synchronize()
    per_kernel = {n: 0.0 for n in names}
    for i in range(cal_steps):
        for j, n in enumerate(names):
            per_kernel[n] += ev.elapsed_ms(marks[i][j], marks[i][j + 1]) / cal_steps
    for m in marks:
        ev.destroy(m)
    dom = max(per_kernel, key=per_kernel.get)
    dj = names.index(dom)

    # timed region: K steps, HIP events around the dominant kernel's launch
    K = args.steps
    starts, stops = ev.create(K), ev.create(K)
    step_marks = []
    for i in range(K):
        m = [None] * (nk + 1)
        m[dj], m[dj + 1] = starts[i], stops[i]
        step_marks.append(m)
    # eager reference result and eager step time (launch by launch from the host)
    y_eager = layer.forward(x).clone()
    torch.cuda.synchronize()
    te0 = time.perf_counter()
    for i in range(K):
        layer.forward_marked(x, y, step_marks[i])
    torch.cuda.synchronize()
    eager_ms = (time.perf_counter() - te0) / K * 1e3

    # each timed step replays a captured HIP graph of one forward (the same kernel
    # launches and event records, replayed without host launch gaps); eager
    # launches when capture is unavailable
    graphs = []
    graph_note = None
    if not args.eager:
        try:
            cs = torch.cuda.Stream()
            for i in range(K):
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=cs):
                    layer.forward_marked(x, y, step_marks[i])
                graphs.append(g)
            torch.cuda.synchronize()
            for g in graphs[:3]:  # replays must reproduce the eager result exactly
                y.zero_()
                g.replay()
                torch.cuda.synchronize()
                if not torch.equal(y.view(torch.int16) if y.dtype == torch.bfloat16 else y,
                                   y_eager.view(torch.int16) if y.dtype == torch.bfloat16 else y_eager):
                    raise RuntimeError("graph replay differs from the eager forward")
        except Exception as ex:  # pragma: no cover - depends on the runtime
            graphs, graph_note = [], f"graph capture unavailable: {ex}"[:200]
    print(f"[bench] timing {K} steps (dominant kernel {dom}, "
          f"{'graph replay' if graphs else 'eager'})", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    if graphs:
        for g in graphs:
            g.replay()
    else:
        for i in range(K):
            layer.forward_marked(x, y, step_marks[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    dom_ms = sum(ev.elapsed_ms(starts[i], stops[i]) for i in range(K)) / K
    ev.destroy(starts)
    ev.destroy(stops)
    elapsed = t1 - t0
    ms_per_step = elapsed / K * 1e3
    value = cfg.tokens * K / elapsed

    work = kernel_work(cfg)
    by, fl, bound = work[dom]
    traffic = None
    tfile = os.path.join(ROOT, "profiles", "traffic.json")
    if os.path.exists(tfile):
        try:
            tj = json.load(open(tfile)).get(f"{wname}:{dom}")
            if tj and tj.get("kernel_source_sha") == bm_kernel_sha(dom, cfg):
                traffic = tj.get("bytes_per_launch")
        except Exception:
            traffic = None
    roof = roofline_entry(by, fl, bound, dom_ms / 1e3, traffic)
    roof["kernel"] = dom
    roof["avg_us"] = round(dom_ms * 1e3, 2)

    kernels = {}
    for n in names:
        b_, f_, bd_ = work[n]
        e = roofline_entry(b_, f_, bd_, per_kernel[n] / 1e3)
        kernels[n] = {"us": round(per_kernel[n] * 1e3, 2), "bound": bd_, "frac": e["frac"]}

    cpu = None
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (fp64 oracle)", file=sys.stderr, flush=True)
        y64 = y.float().cpu().numpy().astype(np.float64)
        cpu = cpu_baseline(inp, y64, args.cpu_seconds)

    out = {
        "metric": "routed tokens/sec per ButterflyMoE layer",
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.act,
        "data": "synthetic (seeded Gaussian activations, uniform ternary substrate, uniform angles)",
        "weight_prep": ({"once_ms": round(prep_ms, 3), "in_timed_steps": False} if prep_ms is not None
                        else {"in_timed_steps": layer.prepared_bytes() > 0}),
        "launch": ({"mode": "graph replay", "eager_ms_per_step": round(eager_ms, 5)} if graphs
                   else {"mode": "eager", "note": graph_note}),
        "config": {"workload": wname, "d_model": cfg.d_model, "d_ff": cfg.d_ff,
                   "n_experts": cfg.n_experts, "top_k": cfg.top_k, "tokens": cfg.tokens,
                   "routed_rows": cfg.tokens * cfg.top_k, "parallelism": "single GPU",
                   "routing": {"gate_mode": "skewed" if args.skewed else "normal", **load}},
        "roofline": roof,
        "cpu_baseline": cpu,
        "kernels": kernels,
    }
    print(json.dumps(out))
    return 0


def bm_kernel_sha(kernel: str, cfg) -> str:
    """Hash of the HIP source that holds `kernel` (to invalidate stale counters)."""
    import hashlib
    g = "gemm_fp4.hip" if cfg.act == "bf16" and cfg.d_model >= 256 else "gemm.hip"
    src = {"gemm": g, "gemm_up": g, "gemm_down": g, "combine": "gemm.hip",
           "route": "route.hip", "bucket": "route.hip", "prep": "prep.hip", "prep_lo": "butterfly_split.hip",
           "prep_hi": "butterfly_split.hip",
           "fused": "fused_mfma.hip"}.get(kernel, "butterfly_split.hip" if kernel.endswith(("_hi", "_lo", "_lo_t"))
                                          else "butterfly.hip")
    p = os.path.join(ROOT, "compressed_mixture_experts_amd", "csrc", src)
    return hashlib.sha256(open(p, "rb").read()).hexdigest()[:16]


if __name__ == "__main__":
    sys.exit(main())
