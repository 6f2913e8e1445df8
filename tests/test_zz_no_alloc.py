"""bmoe_forward_noalloc (include/bmoe.h) against bmoe_forward on the GPU.

The allocation-free entry runs the same kernels as bmoe_forward with the
library's fixed device scratch as the workspace, so its outputs must equal
bmoe_forward's bit for bit (routing indices, gates and y).  Each case makes
two calls in a row on the shared scratch, the second with fewer tokens, so a
stale scratch from the first call would show."""
import numpy as np
import pytest

import compressed_mixture_experts_amd as bm
from compressed_mixture_experts_amd import workloads as wl
from gpu_helpers import log, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _cuda():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    bm.lib()
    yield


CASES = [
    # the edge layer with prepared weights, then 1000 of its tokens
    (dict(cfg=1), True, (4096, 1000)),
    # an FFN layer with split rotations, weights prepared inside every call
    (dict(d_model=1024, d_ff=2048, n_experts=8, top_k=2, tokens=600, act="bf16"), False, (600, 77)),
    # fp32 layer, top-3 with renormalised gates
    (dict(d_model=128, n_experts=6, top_k=3, tokens=500, act="f32", renorm_gates=True), False, (500, 31)),
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_noalloc_matches_forward(case):
    import torch
    kw, prepared, sizes = CASES[case]
    cfg = wl.CONFIGS[kw["cfg"]] if "cfg" in kw else wl.small_config(seed_index=800 + case, **kw)
    inp = wl.generate(cfg)
    layer = bm.Layer.from_inputs(inp, device="cuda")
    if prepared:
        layer.prepare()
    x_all = to_dev(inp.x, cfg.act)
    for T in sizes:
        log(f"noalloc {cfg.name} prepared={prepared} T={T}")
        x = x_all[:T].contiguous()
        y0, i0, g0 = layer.forward(x, return_routing=True)
        y1 = torch.full_like(x, float("nan"))
        i1 = torch.full((T, cfg.top_k), -7, dtype=torch.int32, device="cuda")
        g1 = torch.full((T, cfg.top_k), float("nan"), dtype=torch.float32, device="cuda")
        layer.forward_noalloc(x, y1, i1, g1)
        torch.cuda.synchronize()
        assert torch.equal(i0, i1) and torch.equal(g0, g1)
        if cfg.act == "bf16":
            assert torch.equal(y0.view(torch.int16), y1.view(torch.int16))
        else:
            assert torch.equal(y0, y1)
    # routing outputs are optional
    y2 = torch.empty_like(x_all[:sizes[1]])
    layer.forward_noalloc(x_all[:sizes[1]].contiguous(), y2)
    torch.cuda.synchronize()
    assert torch.equal(y2.view(torch.int16) if cfg.act == "bf16" else y2,
                       y0.view(torch.int16) if cfg.act == "bf16" else y0)


def test_noalloc_rejects_a_workspace_beyond_the_scratch():
    import torch
    cfg = wl.small_config(d_model=512, n_experts=64, top_k=2, tokens=40000, act="bf16", seed_index=810)
    inp = wl.generate(cfg)
    layer = bm.Layer.from_inputs(inp, device="cuda")
    x = to_dev(inp.x, cfg.act)
    y = torch.empty_like(x)
    log("noalloc oversized")
    with pytest.raises(bm.BmoeError) as e:
        layer.forward_noalloc(x, y)
    assert e.value.name == "BMOE_ERR_WORKSPACE"
    # the scratch still serves a fitting call afterwards
    y0 = layer.forward(x[:2000].contiguous())
    y1 = torch.empty_like(y0)
    layer.forward_noalloc(x[:2000].contiguous(), y1)
    torch.cuda.synchronize()
    assert torch.equal(y0.view(torch.int16), y1.view(torch.int16))
