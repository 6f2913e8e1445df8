"""Shared helpers of the GPU parity tests (upload, download, error metrics)."""
import sys

import numpy as np

import compressed_mixture_experts_amd as bm
from compressed_mixture_experts_amd import workloads as wl


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(a, act):
    import torch
    if act == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint16).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def to_f64(t):
    """Exact float64 value of a device tensor (bf16 or fp32)."""
    import torch
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.float().numpy().astype(np.float64)
    return t.numpy().astype(np.float64)


def row_rel_err(y, ref):
    """Per-row relative L2 error ||y - ref|| / ||ref||."""
    num = np.linalg.norm(y - ref, axis=1)
    den = np.maximum(np.linalg.norm(ref, axis=1), 1e-30)
    return num / den


def tol_for(act):
    return 1e-4 if act == "f32" else 2e-2


def run_layer(inp, return_routing=True, prepared=False):
    import torch
    layer = bm.Layer.from_inputs(inp, device="cuda")
    if prepared:
        layer.prepare()
    x = to_dev(inp.x, inp.cfg.act)
    out = layer.forward(x, return_routing=return_routing)
    torch.cuda.synchronize()
    return layer, x, out


def abs_butterfly_apply(angles, M, transpose=False):
    """|S_{L-1}| ... |S_0| M (or the transposed order for B^T): the butterfly of
    the given angles applied stage by stage with |cos| and |sin| in place of
    cos and sin, M [n][m] non-negative.  Elementwise it bounds |B| |M|, since
    each Givens block of B = S_{L-1} ... S_0 is a product of the stages' blocks
    (triangle inequality); used for forward error bounds of rotations computed
    in steps with rounding."""
    ang = np.asarray(angles, dtype=np.float64)
    L = ang.shape[0]
    n = 1 << L
    V = np.array(M, dtype=np.float64, copy=True)
    for s in (range(L - 1, -1, -1) if transpose else range(L)):
        h = 1 << s
        c = np.abs(np.cos(ang[s])).reshape(n // (2 * h), h, 1)
        sn = np.abs(np.sin(ang[s])).reshape(n // (2 * h), h, 1)
        W = V.reshape(n // (2 * h), 2, h, V.shape[1])
        a, b = W[:, 0].copy(), W[:, 1].copy()
        W[:, 0] = c * a + sn * b
        W[:, 1] = sn * a + c * b
        V = W.reshape(n, -1)
    return V
