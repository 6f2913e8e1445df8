"""Seeded synthetic workloads for the ButterflyMoE expert layer.

This module only draws random numbers and rounds them to the stored dtypes.
It holds none of the layer's arithmetic: the fp64 checker and the HIP path
both take its arrays as their inputs.

Workload shapes and value distributions follow the layer settings that the
ButterflyMoE summaries describe (gist.science/*/paper/2601.13563: technical
summary, "Methodology" and "Results" sections, d=512 with 64 and 256 experts)
and the ButterflyViT FFN form (gist.science/pt/paper/2603.06746, "Metodologia").
The pages' own datasets (WikiText, CIFAR-100) are replaced by i.i.d. Gaussian
activations of the same width.

Array conventions (all numpy, C-contiguous):
  x        [T][d_model]             float32, or uint16 holding bf16 bits
  w_gate   [n_experts][d_model]     same dtype as x (one gate vector per expert)
  w_base   list of int8 [d_out][d_in] with values in {-1, 0, +1}
           square layer: [W]          (d x d)
           FFN layer:    [W_up, W_dn] (d_ff x d, d x d_ff)
  theta    list of float32 [N][log2 d_in][d_in/2]   input-side angles
  phi      list of float32 [N][log2 d_out][d_out/2] output-side angles
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Optional

import numpy as np

_SEED_BASE = 0xB7F1


@dataclasses.dataclass(frozen=True)
class LayerConfig:
    name: str
    d_model: int
    d_ff: int            # 0 => square experts (one substrate d x d)
    n_experts: int
    top_k: int
    tokens: int
    act: str             # "f32" or "bf16"
    ffn_act: str = "none"        # "none" or "gelu" (exact erf form)
    outlier_frac: float = 0.0    # fraction of channels scaled (fixed by seed)
    outlier_scale: float = 1.0
    renorm_gates: bool = False
    w_scale: float = 1.0
    seed_index: int = 0

    @property
    def is_ffn(self) -> bool:
        return self.d_ff > 0

    def substrate_shapes(self):
        """(d_out, d_in) of each shared ternary substrate."""
        if self.is_ffn:
            return [(self.d_ff, self.d_model), (self.d_model, self.d_ff)]
        return [(self.d_model, self.d_model)]

    def with_tokens(self, tokens: int) -> "LayerConfig":
        return dataclasses.replace(self, tokens=tokens)


# The five layer settings, in order: tiny check layer, the pages' d=512 edge
# layer with 64 experts, the 256-expert scaling point, a ViT-style FFN MoE, and
# a large FFN layer with activation outliers.
CONFIGS: List[LayerConfig] = [
    LayerConfig("tiny_d64_n4_top1", 64, 0, 4, 1, 16, "f32", seed_index=0),
    LayerConfig("edge_d512_n64_top2", 512, 0, 64, 2, 4096, "bf16", seed_index=1),
    LayerConfig("scale_d512_n256_top2", 512, 0, 256, 2, 16384, "bf16", seed_index=2),
    LayerConfig("vit_ffn_d1024_f4096_n64_top2", 1024, 4096, 64, 2, 8192, "bf16",
                ffn_act="gelu", seed_index=3),
    LayerConfig("large_ffn_d2048_f8192_n256_top2_outliers", 2048, 8192, 256, 2,
                32768, "bf16", ffn_act="gelu", outlier_frac=0.01,
                outlier_scale=50.0, seed_index=4),
]

BENCH_CONFIG_INDEX = 4


@dataclasses.dataclass
class LayerInputs:
    cfg: LayerConfig
    x: np.ndarray
    w_gate: np.ndarray
    w_base: List[np.ndarray]
    theta: List[np.ndarray]
    phi: List[np.ndarray]
    outlier_channels: Optional[np.ndarray] = None


def round_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float values to bf16 (round-to-nearest-even on the float32 value).

    Values are first rounded to float32, then the float32 bit pattern is rounded
    to its upper 16 bits with ties to even.  Returns uint16 bit patterns.
    """
    f = np.ascontiguousarray(a, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)
    # NaN stays NaN (not produced by these generators, kept for safety)
    nan = np.isnan(f)
    if nan.any():
        r[nan] = 0x7FC0
    return r


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32 (for host-side display)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _store(a64: np.ndarray, act: str) -> np.ndarray:
    if act == "f32":
        return np.ascontiguousarray(a64, dtype=np.float32)
    if act == "bf16":
        return round_to_bf16_bits(a64)
    raise ValueError(f"unknown act dtype {act!r}")


def _angles(rng: np.random.Generator, n_experts: int, n: int, mode: str) -> np.ndarray:
    L = int(math.log2(n))
    shape = (n_experts, L, n // 2)
    if mode == "uniform":
        a = rng.uniform(-math.pi, math.pi, size=shape)
    elif mode == "zero":
        a = np.zeros(shape)
    elif mode == "pi":
        a = np.full(shape, math.pi)
    elif mode == "half_pi":
        a = np.full(shape, math.pi / 2)
    elif mode == "quarter_pi":
        a = np.full(shape, math.pi / 4)
    elif mode == "small":
        a = rng.uniform(-1e-3, 1e-3, size=shape)
    else:
        raise ValueError(mode)
    return np.ascontiguousarray(a, dtype=np.float32)


def generate(cfg: LayerConfig, *, angle_mode: str = "uniform", x_mode: str = "normal",
             gate_mode: str = "normal", seed_index: Optional[int] = None) -> LayerInputs:
    """Draw one seeded set of layer inputs for ``cfg``.

    Streams: SeedSequence((0xB7F1, seed_index)).spawn(6) gives independent
    generators for [x, w_gate, w_base[0], w_base[1], angles, outlier channels].
    Draws are float64 and rounded once to the stored dtype.

    x_mode:    "normal"  x ~ N(0, 1)
               "integer" x uniform integers in [-8, 8] (exact in bf16)
    gate_mode: "normal"  w_gate ~ N(0, 1/d_model)
               "skewed"  row e scaled by 4/(e+1)^0.75: a few experts take most of
                         the load, many get few or no tokens
    angle_mode: "uniform" U[-pi, pi); or the closed-form cases "zero", "pi",
               "half_pi", "quarter_pi", "small".
    """
    si = cfg.seed_index if seed_index is None else seed_index
    ss = np.random.SeedSequence((_SEED_BASE, si))
    r_x, r_g, r_w0, r_w1, r_a, r_o = [np.random.default_rng(s) for s in ss.spawn(6)]
    d, N, T = cfg.d_model, cfg.n_experts, cfg.tokens

    if x_mode == "normal":
        x64 = r_x.standard_normal((T, d))
    elif x_mode == "integer":
        x64 = r_x.integers(-8, 9, size=(T, d)).astype(np.float64)
    else:
        raise ValueError(x_mode)
    outliers = None
    if cfg.outlier_frac > 0.0:
        n_out = int(round(cfg.outlier_frac * d))
        outliers = np.sort(r_o.choice(d, size=n_out, replace=False))
        x64[:, outliers] *= cfg.outlier_scale

    g64 = r_g.standard_normal((N, d)) / math.sqrt(d)
    if gate_mode == "skewed":
        # popularity skew: wider logits win the top-k more often, so scaling
        # expert e's gate row by 4 / (e+1)^0.75 gives the low experts most of
        # the load and leaves high ones with few or no tokens
        g64 = g64 * (4.0 / (np.arange(N)[:, None] + 1.0) ** 0.75)
    elif gate_mode != "normal":
        raise ValueError(gate_mode)

    w_base = []
    for m, (d_out, d_in) in enumerate(cfg.substrate_shapes()):
        rng = r_w0 if m == 0 else r_w1
        w_base.append(np.ascontiguousarray(rng.integers(-1, 2, size=(d_out, d_in)), dtype=np.int8))

    theta, phi = [], []
    for (d_out, d_in) in cfg.substrate_shapes():
        theta.append(_angles(r_a, N, d_in, angle_mode))
        phi.append(_angles(r_a, N, d_out, angle_mode))

    return LayerInputs(cfg=cfg, x=_store(x64, cfg.act), w_gate=_store(g64, cfg.act),
                       w_base=w_base, theta=theta, phi=phi, outlier_channels=outliers)


def small_config(d_model=64, d_ff=0, n_experts=4, top_k=2, tokens=37, act="bf16",
                 ffn_act=None, renorm_gates=False, w_scale=1.0, seed_index=100,
                 outlier_frac=0.0, outlier_scale=1.0) -> LayerConfig:
    """A reduced layer for parity tests (several tiles and a ragged tail)."""
    if ffn_act is None:
        ffn_act = "gelu" if d_ff > 0 else "none"
    return LayerConfig(f"small_d{d_model}_f{d_ff}_n{n_experts}_k{top_k}_t{tokens}_{act}",
                       d_model, d_ff, n_experts, top_k, tokens, act, ffn_act=ffn_act,
                       outlier_frac=outlier_frac, outlier_scale=outlier_scale,
                       renorm_gates=renorm_gates, w_scale=w_scale, seed_index=seed_index)
