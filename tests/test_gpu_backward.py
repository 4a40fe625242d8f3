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


# ---------------------------------------------------------------------------
# Token tiles, weight gradients, SwiGLU backward, gate and router gradients
# ---------------------------------------------------------------------------

def _rows_layout(qt, cho, offsets, n_rows):
    """The GPU's transposed tile codes qt [C][P] back in row layout [rows][C]
    (row r of group g, tile j at column 128 (cho[g] + j) + (r - first row of
    the tile)); also checks that padded rows hold code 0."""
    C = qt.shape[0]
    out = np.zeros((n_rows, C), np.uint8)
    for g in range(len(offsets) - 1):
        for j, r0 in enumerate(range(offsets[g], offsets[g + 1], 128)):
            r1 = min(r0 + 128, offsets[g + 1])
            col = 128 * (cho[g] + j)
            out[r0:r1] = qt[:, col:col + r1 - r0].T
            assert np.all(qt[:, col + r1 - r0:col + 128] == 0)
    return out


@pytest.mark.parametrize("src_dtype", [torch.bfloat16, torch.float32])
def test_quant_tokens_bit_exact(src_dtype):
    """Groups of 0, 1, 127, 128, 129, 300 rows gathered from a source matrix,
    with and without a per-row multiplier: codes, scales and the groups'
    tile offsets bit for bit against the oracle."""
    d = _d()
    r = np.random.default_rng(12)
    sizes = [0, 1, 127, 128, 129, 300]
    offsets = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64)
    m = int(offsets[-1])
    n_src, C = 400, 384
    src = normal_bf16("gtok_src", (n_src, C), 1.0, seed=3)
    src[7, 5] = np.float32(300.0)              # an outlier
    if src_dtype == torch.float32:
        src = (src * np.float32(1.0 + 2.0 ** -12)).astype(np.float32)   # not bf16-representable
    rows = r.integers(0, n_src, m).astype(np.int32)
    gate = (r.random(m) * 0.9 + 0.05).astype(np.float32)
    off_d = torch.tensor(offsets, dtype=torch.int32, device="cuda")
    for with_scale in (False, True):
        banner(f"quant_tokens {src_dtype} row_scale={with_scale}")
        qt, sc, cho = d.quant_tokens_128(dev(src, src_dtype), off_d, m_total=m,
                                         rows=dev(rows), row_scale=dev(gate) if with_scale else None)
        v = src[rows] * gate[:, None] if with_scale else src[rows]    # float32 products, rounded once
        q_o, s_o = ob.quant_tokens_128(v.astype(np.float32), offsets)
        cho_h = host(cho)
        assert np.array_equal(cho_h, ob.chunk_offsets(offsets))
        n_t = int(cho_h[-1])
        assert np.array_equal(host(sc)[:n_t].view(np.uint32), s_o.view(np.uint32))
        assert np.array_equal(_rows_layout(host(qt), cho_h, offsets.tolist(), m), q_o)


def _wgrad_case(M, N, sizes, out_dtype, seed, what):
    d = _d()
    offsets = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64)
    m = int(offsets[-1])
    dc = normal_bf16("gwg_dc", (m, M), 1.0, seed=seed)
    a = normal_bf16("gwg_a", (m, N), 1.0, seed=seed + 1)
    banner(f"wgrad {what}: M={M} N={N} groups {sizes} {out_dtype}")
    off_d = torch.tensor(offsets, dtype=torch.int32, device="cuda")
    qg, sg, cho = d.quant_tokens_128(dev(dc, torch.bfloat16), off_d)
    qa, sa, _ = d.quant_tokens_128(dev(a, torch.bfloat16), off_d)
    c = d.fp8_wgrad_grouped(qg, sg, qa, sa, cho, out_dtype=out_dtype)
    qg_o, sg_o = ob.quant_tokens_128(dc, offsets)
    qa_o, sa_o = ob.quant_tokens_128(a, offsets)
    want, norm = ob.wgrad_grouped(qg_o, sg_o, qa_o, sa_o, offsets)
    tol = 2e-3 if out_dtype == torch.float32 else 1e-2
    assert_normalised_close(host(c), want, norm, tol, f"wgrad {what}")


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_wgrad_grouped_ragged_groups(out_dtype):
    """Empty groups (zero gradient), one row, a tile and a bit, three tiles."""
    _wgrad_case(256, 384, [0, 1, 129, 0, 300, 64], out_dtype, 21, "ragged")


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_wgrad_grouped_column_tile_runs(out_dtype):
    """11 column tiles, which a block takes 8 at a time (a full run and a run
    of 3), over empty groups, one row, two token tiles and a whole tile."""
    _wgrad_case(256, 1408, [0, 130, 1, 0, 257, 128], out_dtype, 23, "column-tile runs")


@pytest.mark.parametrize("M,N,split", [(1024, 512, "8 x 1"), (1024, 2048, "2 x 4"), (2048, 1024, "4 x 2")])
def test_wgrad_grouped_xcd_splits(M, N, split):
    """Shapes whose (row tile, column run) pairs the launch splits over the
    XCDs as 8 x 1, 2 x 4 and 4 x 2 parts, over ragged and empty groups."""
    _wgrad_case(M, N, [130, 0, 1, 257, 64], torch.float32, M + 3 * N, f"xcd split {split}")


@pytest.mark.parametrize("M,N,what", [(7168, 2048, "dW2 of a V3 expert"), (4096, 7168, "dW13 of a V3 expert")])
def test_wgrad_v3_shapes(M, N, what):
    """One V3 expert with 300 rows (three token tiles): dW2 [7168][2048] and
    dW13 [4096][7168]."""
    _wgrad_case(M, N, [300], torch.float32, M + N, what)


def test_swiglu_backward_against_oracle():
    """Same float32 inputs on both sides: dh within a few float32 ulps of the
    float64 derivative, relative to the size of its terms (1 + g (1 - sig)
    cancels near g = -1.28, so the bound is taken on the terms)."""
    d = _d()
    r = np.random.default_rng(13)
    rows, inter = 300, 384
    h = (r.standard_normal((rows, 2 * inter)) * 3.0).astype(np.float32)
    h[0, :inter] = 0.0
    da = r.standard_normal((rows, inter)).astype(np.float32)
    gate = (r.random(rows) * 0.9 + 0.05).astype(np.float32)
    banner("swiglu backward")
    dh, a = d.swiglu_backward(dev(h), dev(da), dev(gate), recompute_a=True)
    dd = (gate[:, None] * da).astype(np.float32).astype(np.float64)     # the kernel's float32 product
    want = ob.swiglu_backward(h, dd)
    g, u = h[:, :inter].astype(np.float64), h[:, inter:].astype(np.float64)
    sig = 1.0 / (1.0 + np.exp(-g))
    norm_g = np.abs(dd * u) * sig * (1.0 + np.abs(g) * (1.0 - sig))
    norm_u = np.abs(dd * g) * sig
    got = host(dh)
    assert_normalised_close(got[:, :inter], want[:, :inter], norm_g, 1e-5, "dh gate")
    assert_normalised_close(got[:, inter:], want[:, inter:], norm_u, 1e-5, "dh up")
    assert_normalised_close(host(a), g * sig * u, np.abs(g * sig * u), 1e-5, "recomputed a")


@pytest.mark.parametrize("o_dtype", [torch.float32, torch.bfloat16])
def test_gate_backward_against_oracle(o_dtype):
    """dgate = <dy, o_k> and the router logits' gradient through the
    normalisation and the sigmoid, against the oracle on the same dy, o and
    logits; each bounded by the float32 evaluation relative to the sizes of
    its terms."""
    from oracle import route as orr
    d = _d()
    r = np.random.default_rng(14)
    T, E, G, Mg, K, H = 70, 64, 8, 4, 8, 1024
    logits = (r.standard_normal((T, E)) * 2.0).astype(np.float32)
    rt = orr.route(logits, np.zeros(E, np.float32), G, Mg, K)
    idx = rt["topk_idx"]
    perm_inv = r.permutation(T * K).astype(np.int32).reshape(T, K)      # any row order
    dy = normal_bf16("ggb_dy", (T, H), 1.0, seed=1)
    o = normal_bf16("ggb_o", (T * K, H), 0.5, seed=2)
    banner(f"gate backward o {o_dtype}")
    dgate, dz = d.gate_backward(dev(dy, torch.bfloat16), dev(o, o_dtype), dev(perm_inv), dev(idx), dev(logits))
    o_tk = o[perm_inv]                                                     # [T][K][H]
    want_g, want_z = ob.gate_backward(dy, o_tk, idx, logits, E)
    dn = np.einsum("th,tkh->tk", np.abs(dy).astype(np.float64), np.abs(o_tk).astype(np.float64))
    assert_normalised_close(host(dgate), want_g, dn, 1e-5, "dgate")
    s = orr.affinity(logits).astype(np.float64)
    s_sel = np.take_along_axis(s, idx.astype(np.int64), axis=1)
    tot = s_sel.sum(axis=1, keepdims=True)
    zn = np.zeros((T, E))
    np.put_along_axis(zn, idx.astype(np.int64),
                      s_sel * (1 - s_sel) * (dn + np.sum(dn * s_sel / tot, axis=1, keepdims=True)) / tot, axis=1)
    assert_normalised_close(host(dz), want_z, zn, 1e-5, "dlogits")


# ---------------------------------------------------------------------------
# The whole expert backward of a layer, chained on the GPU
# ---------------------------------------------------------------------------

def _row_gates(gates, inv, n_rows):
    """Gate of each (token, expert) row: row inv[t][k] carries gates[t][k]."""
    g = np.zeros(n_rows, np.float32)
    g[inv.reshape(-1)] = gates.reshape(-1)
    return g


def test_layer_backward_chain_against_oracle():
    """Forward on the GPU, then the whole FP8 expert backward chained through
    the C ABI (recomputed h and o, gate and router-logit gradients, the dgrad
    of the down projection, the SwiGLU backward, the dgrad of the gate/up
    projection summed per token, and both weight gradients of every routed
    expert and the shared one), against the oracle's chain in float64.

    As in the forward's protocol, a step whose FP8 input is quantised from a
    float32 intermediate (a for dW2, dh for the gate/up dgrad and dW13) runs
    in the oracle on the GPU's intermediate, once that intermediate has been
    checked against the oracle's own: a value within float32 rounding of an
    E4M3 rounding point has more than one valid code, and a short contraction
    (an expert's tokens) does not average such a difference away.  Every
    check: max |gpu - oracle| / D <= 2e-3, D the normaliser of the step
    (for dh and a, the first-order sensitivity to their inputs' normalisers)."""
    from oracle import gemm as og
    from dsmoe_inputs import LayerConfig, layer_inputs_host
    d = _d()
    cfg = LayerConfig("bwd", T=300, H=512, E=16, G=4, Mg=2, K=4, I=256, router_std=0.02, bias_range=0.01)
    T, H, E, K, I = cfg.T, cfg.H, cfg.E, cfg.K, cfg.I
    inp = layer_inputs_host(cfg, 0)
    banner(f"layer backward chain T={T} H={H} E={E} K={K} I={I}")
    x = dev(inp["x"], torch.bfloat16)
    w13d, w2d = dev(inp["w13"], torch.bfloat16), dev(inp["w2"], torch.bfloat16)
    weights = d.quantize_layer_weights(w13d[:E], w2d[:E], dev(inp["router_w"], torch.bfloat16), w13d[E], w2d[E])
    desc = d.MoEDesc(H, I, E, cfg.G, cfg.Mg, K, 1)
    _, counts, g = d.moe_forward(desc, weights, dev(inp["bias"]), x, out_dtype=torch.float32, debug=True)
    q13, s13 = d.quant_w_128x128(w13d)          # E + 1 groups, the shared expert last
    q2, s2 = d.quant_w_128x128(w2d)
    wt = d.transpose_w_128x128(q13, s13) + d.transpose_w_128x128(q2, s2)
    dy_h = normal_bf16("bwd_dy", (T, H), 1.0, seed=9)
    dy = dev(dy_h, torch.bfloat16)
    out = d.moe_backward_experts(g, x, dy, (q13, s13, q2, s2), wt, T, K)
    gh = {k: host(v) for k, v in g.items()}
    oh = {k: host(v) for k, v in out.items()}

    # the oracle's chain on the same routing (GPU logits) and codes of a
    q13o, s13o = oq.quant_w_128x128(inp["w13"])
    q2o, s2o = oq.quant_w_128x128(inp["w2"])
    assert np.array_equal(host(q13), q13o) and np.array_equal(host(q2), q2o)
    rows = T * K + T
    off = np.concatenate([gh["offsets"], [rows]]).astype(np.int64)
    perm = np.concatenate([gh["perm"], np.arange(T)]).astype(np.int64)
    rg = _row_gates(gh["gates"], gh["inv"], rows)
    rg[T * K:] = 1.0
    qx, sx = oq.quant_act_1x128(inp["x"])
    h_or, h_d = og.grouped_gemm(qx, sx, perm, off, q13o, s13o)
    assert_normalised_close(oh["h"], h_or, h_d, 2e-3, "chain recomputed h")
    o_or, o_d = og.grouped_gemm(gh["qa"], gh["sa"], None, off, q2o, s2o)
    assert_normalised_close(oh["o"], o_or, o_d, 2e-3, "chain recomputed o")
    dgate, dz = ob.gate_backward(dy_h, o_or[gh["inv"]], gh["topk_idx"], gh["logits"], E)
    dn = np.einsum("th,tkh->tk", np.abs(dy_h).astype(np.float64), o_d[gh["inv"]])
    assert_normalised_close(oh["dgate"], dgate, dn, 2e-3, "chain dgate")
    s = 1.0 / (1.0 + np.exp(-gh["logits"].astype(np.float64)))
    s_sel = np.take_along_axis(s, gh["topk_idx"].astype(np.int64), axis=1)
    tot = s_sel.sum(axis=1, keepdims=True)
    zn = np.zeros((T, E))
    np.put_along_axis(zn, gh["topk_idx"].astype(np.int64),
                      s_sel * (1 - s_sel) * (dn + np.sum(dn * s_sel / tot, axis=1, keepdims=True)) / tot, axis=1)
    assert_normalised_close(oh["dlogits"], dz, zn, 2e-3, "chain dlogits")

    qdy, sdy = oq.quant_act_1x128(dy_h)
    da, da_d = ob.dgrad_grouped(qdy, sdy, perm, off, q2o, s2o)
    assert_normalised_close(oh["da"], da, da_d, 2e-3, "chain dgrad of the down projection")
    # SwiGLU backward: first-order sensitivity of dh and a to h and da
    dd, dd_d = rg[:, None] * da, rg[:, None] * da_d
    dh = ob.swiglu_backward(h_or, dd)
    gg, uu = h_or[:, :I], h_or[:, I:]
    gd, ud = h_d[:, :I], h_d[:, I:]
    sig = 1.0 / (1.0 + np.exp(-gg))
    silu = gg * sig
    n_g = 1.1 * np.abs(uu) * dd_d + 1.1 * np.abs(dd) * ud + 0.5 * np.abs(dd * uu) * gd
    n_u = np.abs(silu) * dd_d + 1.1 * np.abs(dd) * gd
    assert_normalised_close(oh["dh"][:, :I], dh[:, :I], n_g, 2e-3, "chain dh gate")
    assert_normalised_close(oh["dh"][:, I:], dh[:, I:], n_u, 2e-3, "chain dh up")
    assert_normalised_close(oh["a"], silu * uu, 1.1 * np.abs(uu) * gd + np.abs(silu) * ud, 2e-3,
                            "chain recomputed a")
    # the steps after the requantisation of dh and a, on the GPU's dh and a
    dh_g, a_g = oh["dh"].astype(np.float32), oh["a"].astype(np.float32)
    qdh, sdh = oq.quant_act_1x128(dh_g)
    dxr, dxr_d = ob.dgrad_grouped(qdh, sdh, None, off, q13o, s13o)
    inv = gh["inv"]
    dx = dxr[T * K:] + sum(dxr[inv[:, k]] for k in range(K))
    dx_d = dxr_d[T * K:] + sum(dxr_d[inv[:, k]] for k in range(K))
    assert_normalised_close(oh["dx"], dx, dx_d, 2e-3, "chain dx (expert path)")
    do = (rg[:, None] * dy_h[perm]).astype(np.float32)
    qdo, sdo = ob.quant_tokens_128(do, off)
    qa_t, sa_t = ob.quant_tokens_128(a_g, off)
    dw2, dw2_d = ob.wgrad_grouped(qdo, sdo, qa_t, sa_t, off)
    assert_normalised_close(oh["dw2"], dw2, dw2_d, 2e-3, "chain dW2")
    qdh_t, sdh_t = ob.quant_tokens_128(dh_g, off)
    qx_t, sx_t = ob.quant_tokens_128(inp["x"][perm], off)
    dw13, dw13_d = ob.wgrad_grouped(qdh_t, sdh_t, qx_t, sx_t, off)
    assert_normalised_close(oh["dw13"], dw13, dw13_d, 2e-3, "chain dW13")
