"""Host-side logic of bench.py (no GPU): the one-GPU contract, the
algorithmic bytes and flops the roofline fractions divide by, and the
fraction arithmetic.

The per-kernel units follow the measurement plan: activations in and out
once, the router's gate matrix once, fp32 angles of the stages a kernel
applies, the ternary substrate at 2 bits per weight, routing indices and
gates; multiply-adds count as 2 flops.  The figures below are worked out by
hand for the edge and large workloads (d, d_ff, N, k, T as in workloads.py).
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from compressed_mixture_experts_amd import workloads as wl  # noqa: E402


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def _cfg(name):
    return next(c for c in wl.CONFIGS if c.name == name)


def test_edge_fused_kernel_bytes_and_flops():
    w = bench.kernel_work(_cfg("edge_d512_n64_top2"))
    T, d, N, k = 4096, 512, 64, 2
    R = T * k
    gathered_x = R * d * 2            # 8,388,608
    per_slot_rows = R * d * 2         # 8,388,608 (the k rows added into y)
    angles = 2 * N * 9 * (d // 2) * 4  # both rotations, 9 stages of 256 pairs: 1,179,648
    substrate = d * d // 4            # 2 bits per weight: 65,536
    slots_gates = 8 * R               # 65,536
    assert w["fused"][0] == gathered_x + per_slot_rows + angles + substrate + slots_gates == 18_087_936
    # substrate product 2 R d^2 plus 3 flops per element per Givens stage, both rotations
    assert w["fused"][1] == 2 * R * d * d + 2 * 3 * R * d * 9
    assert w["fused"][2] == "hbm"     # 250 flop/byte, below the 312.5 ridge
    # top-2: no combine; the bucketing kernel also zeroes y
    assert w["bucket"][0] == 8 * R + 4 * (N + 1) + T * d * 2
    assert w["route"][0] == T * d * 2 + N * d * 2 + 8 * R
    assert w["route"][1] == 2 * T * d * N
    assert set(w) == {"route", "bucket", "fused"}


def test_large_ffn_kernel_bytes_and_flops():
    w = bench.kernel_work(_cfg("large_ffn_d2048_f8192_n256_top2_outliers"))
    T, d, f, N, k = 32768, 2048, 8192, 256, 2
    R = T * k
    # each substrate product: rows in and out once, the shared 2-bit substrate
    # once; the up product's epilogue also applies stages 0..7 of phi_up (their
    # angles, 3 flops per element per stage)
    up = (R * d * 2 + R * f * 2 + f * d // 4, 2 * R * d * f)
    epi = (N * 8 * (f // 2) * 4, 3 * R * f * 8)
    assert w["gemm_up"][:2] == (up[0] + epi[0], up[1] + epi[1])
    assert w["gemm_down"][:2] == (R * f * 2 + R * d * 2 + d * f // 4, 2 * R * f * d)
    assert up[1] == 2_199_023_255_552 and w["gemm_up"][2] == "mfma"
    # low part of theta_dn (width 8192): one pass over the rows, angles of stages 0..8
    assert w["bfly_mid_lo_t"][0] == 2 * R * f * 2 + N * 9 * (f // 2) * 4
    # the FFN middle's pass: stage 8 of phi_up, then the top four stages of
    # both butterflies
    assert w["bfly_mid_hi"][0] == 2 * R * f * 2 + 2 * N * 4 * (f // 2) * 4 + N * (f // 2) * 4
    assert w["bfly_mid_hi"][1] == 3 * R * f * 9
    # output rotation (width 2048, one pass): rows in and out, all 11 stages'
    # angles, slots and gates
    assert w["bfly_out"][0] == 2 * R * d * 2 + N * 11 * (d // 2) * 4 + 8 * R
    assert w["bfly_in"][0] == 2 * R * d * 2 + N * 11 * (d // 2) * 4 + 4 * R
    assert w["combine"][0] == R * d * 2 + T * d * 2 == 402_653_184
    assert w["route"][0] == T * d * 2 + N * d * 2 + 8 * R
    names = ["route", "bucket", "bfly_in", "gemm_up", "bfly_mid_hi",
             "bfly_mid_lo_t", "gemm_down", "bfly_out", "combine"]
    assert set(w) == set(names)


@pytest.mark.parametrize("name", [c.name for c in wl.CONFIGS[1:]])
def test_every_bf16_workload_has_a_bound_per_kernel(name):
    w = bench.kernel_work(_cfg(name))
    for kname, (by, fl, bound) in w.items():
        assert by > 0 and fl >= 0, kname
        ridge = bench.MFMA_BF16_PEAK_TFLOPS / bench.HBM_PEAK_GBS * 1e3
        if kname.startswith("gemm") or kname == "fused":
            assert bound == ("mfma" if fl / by > ridge else "hbm"), kname


def test_roofline_fraction_arithmetic():
    # 2.5 TFLOP in 1 ms is the bf16 matrix-core peak; 8 GB in 1 ms the HBM peak
    e = bench.roofline_entry(1e9, 2.5e12, "mfma", 1e-3)
    assert e["unit"] == "TFLOP/s" and e["achieved"] == 2500.0 and e["frac"] == 1.0
    e = bench.roofline_entry(4e9, 0, "hbm", 1e-3, traffic=123)
    assert e["unit"] == "GB/s" and e["achieved"] == 4000.0 and e["frac"] == 0.5 and e["traffic"] == 123
