"""GPU parity of the data-gradient pieces of the FP8 backward against
oracle.backward: the block transpose of FP8 weights bit for bit, and the
data-gradient grouped GEMM dA = dC . W (dsmoe_fp8_grouped_gemm on the
transposed weights) to the GEMM bar, max |gpu - oracle| / D <= 2e-3 (f32)."""

import numpy as np
import pytest
import torch

from dsmoe_inputs import normal_bf16
from gpu_util import assert_normalised_close, banner, dev, host
from oracle import backward as ob
from oracle import quant as oq

pytestmark = pytest.mark.gpu


def _d():
    import fp8_block_scaled_dsmoe_amd as d
    return d


@pytest.mark.parametrize("shape", [(1, 128, 128), (3, 256, 384), (1, 7168, 2048), (1, 4096, 7168)])
def test_transpose_is_exact(shape):
    banner(f"transpose_w {shape}")
    r = np.random.default_rng(sum(shape))
    q = r.integers(0, 256, shape, dtype=np.uint8)
    s = r.random((shape[0], shape[1] // 128, shape[2] // 128)).astype(np.float32)
    qt, st = _d().transpose_w_128x128(dev(q), dev(s))
    assert np.array_equal(host(qt), np.swapaxes(q, 1, 2))
    assert np.array_equal(host(st).view(np.uint32), np.swapaxes(s, 1, 2).view(np.uint32))


def test_transposed_codes_equal_quantising_the_transpose():
    banner("transpose invariance on the GPU")
    w = normal_bf16("gbwd_w", (2, 256, 384), 0.02, seed=2)
    w[0, 5, 300] = np.float32(1.5)
    d = _d()
    q, s = d.quant_w_128x128(dev(w, torch.bfloat16))
    qt, st = d.transpose_w_128x128(q, s)
    qo, so = d.quant_w_128x128(dev(np.ascontiguousarray(np.swapaxes(w, 1, 2)), torch.bfloat16))
    assert torch.equal(qt, qo) and torch.equal(st, so)


def _dgrad_case(G, N, K, rows, offsets, n_src, seed, what):
    """dC [n_src][N] (gathered by `rows` into groups), W [G][N][K]: dA [M][K]."""
    d = _d()
    w = normal_bf16("gbwd_wg", (G, N, K), 0.02, seed=seed)
    dc = normal_bf16("gbwd_dc", (n_src, N), 1.0, seed=seed + 1)
    banner(f"dgrad {what}: G={G} N={N} K={K} rows={len(rows)}")
    qw, sw = d.quant_w_128x128(dev(w, torch.bfloat16))
    qt, st = d.transpose_w_128x128(qw, sw)
    qg, sg = d.quant_act_1x128(dev(dc, torch.bfloat16))
    off = torch.tensor(offsets, dtype=torch.int32, device="cuda")
    a_rows = torch.tensor(rows, dtype=torch.int32, device="cuda")
    c = d.fp8_grouped_gemm(qg, sg, off, qt, st, out_dtype=torch.float32, a_rows=a_rows)
    qw_o, sw_o = oq.quant_w_128x128(w)
    qg_o, sg_o = oq.quant_act_1x128(dc)
    assert np.array_equal(host(qg), qg_o)
    want, norm = ob.dgrad_grouped(qg_o, sg_o, np.asarray(rows), offsets, qw_o, sw_o)
    assert_normalised_close(host(c), want, norm, 2e-3, f"dgrad {what}")


def test_dgrad_grouped_with_gather_and_ragged_groups():
    r = np.random.default_rng(7)
    rows = r.integers(0, 50, 170).tolist()
    _dgrad_case(G=4, N=256, K=384, rows=rows, offsets=[0, 3, 3, 130, 170], n_src=50, seed=11,
                what="gathered")


@pytest.mark.parametrize("N,K,what", [(7168, 2048, "down projection (dy . W2)"),
                                      (4096, 7168, "gate/up projection (dh . W13)")])
def test_dgrad_v3_shapes(N, K, what):
    """One V3 expert: W2 [7168][2048] (the gradient of the down projection
    contracts over H = 7168) and W13 [4096][7168] (over 2I = 4096)."""
    rows = list(range(200))
    _dgrad_case(G=1, N=N, K=K, rows=rows, offsets=[0, 200], n_src=200, seed=N, what=what)
