"""GPU check of dsmoe_moe_forward_noalloc (the forward on the library's own
device scratch) against dsmoe_moe_forward (the forward on a caller
workspace): the same kernels on the same inputs, so y and the counts must be
identical bit for bit.  Two calls in a row, the second on fewer tokens, so
that the second runs on scratch the first left behind; then the first size
again."""

import numpy as np
import pytest
import torch

from dsmoe_inputs import LAYER_CONFIGS, LayerConfig, layer_inputs_host
from gpu_util import banner, dev

pytestmark = pytest.mark.gpu


def _setup(cfg):
    import fp8_block_scaled_dsmoe_amd as d
    inp = layer_inputs_host(cfg, 0)
    w13 = dev(inp["w13"], torch.bfloat16)
    w2 = dev(inp["w2"], torch.bfloat16)
    weights = d.quantize_layer_weights(w13[:cfg.E], w2[:cfg.E], dev(inp["router_w"], torch.bfloat16),
                                       w13[cfg.E], w2[cfg.E])
    desc = d.MoEDesc(cfg.H, cfg.I, cfg.E, cfg.G, cfg.Mg, cfg.K, 1)
    return d, inp, weights, desc


@pytest.mark.parametrize("cfg,sizes", [
    (LAYER_CONFIGS["tiny"], (256, 100, 256)),
    (LayerConfig("mid", T=1024, H=1024, E=64, G=8, Mg=4, K=8, I=512, router_std=0.02, bias_range=0.01),
     (1024, 300, 1024)),
], ids=["tiny", "mid"])
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_noalloc_forward_matches_workspace_forward(cfg, sizes, out_dtype):
    d, inp, weights, desc = _setup(cfg)
    bias = dev(inp["bias"])
    x_all = dev(inp["x"], torch.bfloat16)
    assert d.moe_workspace_bytes(desc, max(sizes)) <= d.NOALLOC_SCRATCH_BYTES
    for T in sizes:
        banner(f"noalloc {cfg.name} T={T} {out_dtype}")
        x = x_all[:T].contiguous()
        y_ref, c_ref, _ = d.moe_forward(desc, weights, bias, x, out_dtype=out_dtype)
        y = torch.empty((T, cfg.H), dtype=out_dtype, device="cuda")
        c = torch.empty((cfg.E,), dtype=torch.int32, device="cuda")
        y.fill_(float("nan"))
        c.fill_(-1)
        d.moe_forward_noalloc(desc, weights, bias, x, y=y, counts=c)
        torch.cuda.synchronize()
        iv = torch.int32 if out_dtype == torch.float32 else torch.int16
        assert torch.equal(y.view(iv), y_ref.view(iv)), f"T={T}: y differs from the workspace forward"
        assert torch.equal(c, c_ref)
        assert int(c.sum()) == T * cfg.K


def test_noalloc_forward_rejects_oversized_call():
    d, inp, weights, _ = _setup(LAYER_CONFIGS["tiny"])
    big = d.MoEDesc(7168, 2048, 256, 8, 4, 8, 1)
    x = torch.zeros((300, 7168), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(RuntimeError, match="DSMOE_ERR_WORKSPACE"):
        d.moe_forward_noalloc(big, weights, torch.zeros(256, device="cuda"), x)
