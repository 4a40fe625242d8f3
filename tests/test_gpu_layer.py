"""GPU parity of dsmoe_moe_forward and dsmoe_moe_forward_serving against the
oracle's layer, under the protocol of layer_parity.py: x codes bit-exact,
logits within the FP32 bound, routing bit-exact on the GPU's logits, the
codes of the requantised SwiGLU output equal to the oracle's wherever they
are not decided within the FP32 error of h, and y against the oracle's down
projections and combine run on the GPU's own codes, with no allowance.

Small configurations check every token.  The DeepSeek-V3-sized layers check
the routing of every token, the codes of a over whole row tiles of several
experts (the tiles the headline kernels run), and y and every code of a on
sampled tokens (all 64 at decode size).
"""

import concurrent.futures
import os

import numpy as np
import pytest
import torch

import layer_parity as lp
from dsmoe_inputs import LAYER_CONFIGS, LayerConfig, expert_weights_device, layer_inputs_host
from gpu_util import banner, dev, host
from oracle import layer as ol
from oracle import quant as oq

pytestmark = pytest.mark.gpu

DT = {torch.float32: "f32", torch.bfloat16: "bf16"}
N_CPU = min(16, os.cpu_count() or 1)


def _dsmoe():
    import fp8_block_scaled_dsmoe_amd as d
    return d


def _ws_tile_rows(rows_hint):
    """The weight-streaming tile height the GEMM dispatcher picks for groups
    of about rows_hint rows (0: the 256 x 256 LDS kernel); restated here so
    that each configuration below can assert which kernel it exercises."""
    want = rows_hint * 11 // 8
    for bm in (16, 32, 64, 96, 128, 160, 176, 192):
        if want <= bm:
            return bm
    return 0


def _gpu(dbg, counts):
    g = {k: host(v) for k, v in dbg.items()}
    g["counts"] = host(counts)
    return g


def _check_perm_valid(g, T, K, E):
    """The GPU's permutation is consistent with its own routing."""
    idx = g["topk_idx"]
    counts = np.bincount(idx.reshape(-1), minlength=E)
    assert np.array_equal(g["counts"], counts)
    assert np.array_equal(g["offsets"], np.concatenate([[0], np.cumsum(counts)]))
    perm, inv, off = g["perm"], g["inv"], g["offsets"]
    assert sorted(inv.reshape(-1).tolist()) == list(range(T * K))
    tok = np.repeat(np.arange(T), K).reshape(T, K)
    assert np.array_equal(perm[inv], tok)
    for e in range(E):
        seg = perm[off[e]:off[e + 1]]
        assert np.all(np.diff(seg) > 0)
        assert np.all(np.any(idx[seg] == e, axis=1))


def _serving(d, desc, weights, counts, n_extra, bias, x, out_dtype):
    """The serving forward with a replica plan from `counts` (n_extra extra
    slots), the slot weights placed from `weights`."""
    slot_first, slot_expert = d.plan_replicas(counts, n_extra)
    slot_w = d.place_layer_replicas(weights, slot_expert)
    y, c, dbg = d.moe_forward_serving(desc, slot_w, slot_first, slot_expert, bias, x,
                                      out_dtype=out_dtype, debug=True)
    return y, c, dbg, slot_first


def _layer_case(cfg: LayerConfig, out_dtype, n_shared=1, seed=0, serving_extra=None):
    d = _dsmoe()
    inp = layer_inputs_host(cfg, seed)
    T, K, E, I = cfg.T, cfg.K, cfg.E, cfg.I
    banner(f"layer {cfg.name} T={T} H={cfg.H} E={E} K={K} I={I} shared={n_shared} {out_dtype}")
    x = dev(inp["x"], torch.bfloat16)
    wr = dev(inp["router_w"], torch.bfloat16)
    w13 = dev(inp["w13"], torch.bfloat16)
    w2 = dev(inp["w2"], torch.bfloat16)
    weights = d.quantize_layer_weights(w13[:E], w2[:E], wr,
                                       w13[E] if n_shared else None, w2[E] if n_shared else None)
    desc = d.MoEDesc(cfg.H, I, E, cfg.G, cfg.Mg, K, n_shared)
    y, counts, dbg = d.moe_forward(desc, weights, dev(inp["bias"]), x, out_dtype=out_dtype, debug=True)

    q13, s13 = oq.quant_w_128x128(inp["w13"])
    q2, s2 = oq.quant_w_128x128(inp["w2"])
    assert np.array_equal(host(weights.w13), q13[:E])
    assert np.array_equal(host(weights.s2).view(np.uint32), s2[:E].view(np.uint32))
    get = lambda e: (q13[e], s13[e], q2[e], s2[e])
    if n_shared:
        shared = get(E)
    else:
        zero13 = np.zeros_like(q13[0]); zero2 = np.zeros_like(q2[0])
        shared = (zero13, np.ones_like(s13[0]), zero2, np.ones_like(s2[0]))

    g = _gpu(dbg, counts)
    _check_perm_valid(g, T, K, E)
    lp.check_routing_all(g, inp["bias"], cfg.G, cfg.Mg, K, E, cfg.name)
    toks = np.arange(T)
    want = ol.moe_layer(inp["x"], inp["router_w"], inp["bias"], get, shared, cfg.G, cfg.Mg, K,
                        logits=g["logits"], h_rel_err=lp.H_REL_ERR,
                        a_codes=lp.gpu_a_codes(g, T, K, toks, n_shared, I))
    lp.check_tokens(g, host(y), want, toks, T, K, n_shared, DT[out_dtype], f"{cfg.name} {DT[out_dtype]}")
    if serving_extra is not None:
        # the decode-serving forward: slots planned from this step's loads, the
        # shared expert as one more routed group; same routing, same protocol
        banner(f"layer {cfg.name} serving: {serving_extra} extra slots")
        y2, c2, dbg2, slot_first = _serving(d, desc, weights, counts, serving_extra, dev(inp["bias"]), x,
                                            out_dtype)
        g2 = _gpu(dbg2, c2)
        for k in ("counts", "topk_idx", "offsets", "perm", "inv", "qx", "sx", "logits"):
            assert np.array_equal(g2[k], g[k]), f"serving {k} differs from the plain forward's"
        n_rep = np.diff(host(slot_first))
        print(f"[serving] slots per expert: max {n_rep.max()}, max rows per slot "
              f"{(g['counts'] / n_rep).max():.1f} (was {g['counts'].max()})", flush=True)
        want2 = ol.moe_layer(inp["x"], inp["router_w"], inp["bias"], get, shared, cfg.G, cfg.Mg, K,
                             logits=g2["logits"], h_rel_err=lp.H_REL_ERR,
                             a_codes=lp.gpu_a_codes(g2, T, K, toks, n_shared, I))
        lp.check_tokens(g2, host(y2), want2, toks, T, K, n_shared, DT[out_dtype],
                        f"{cfg.name} serving {DT[out_dtype]}")
    return y, counts, g


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_tiny_layer(out_dtype):
    _layer_case(LAYER_CONFIGS["tiny"], out_dtype)


def test_tiny_layer_deterministic():
    cfg = LAYER_CONFIGS["tiny"]
    y1, c1, _ = _layer_case(cfg, torch.float32)
    y2, c2, _ = _layer_case(cfg, torch.float32)
    assert torch.equal(y1.view(torch.int32), y2.view(torch.int32))
    assert torch.equal(c1, c2)


@pytest.mark.parametrize("cfg", [
    LayerConfig("ragged", T=77, H=256, E=8, G=2, Mg=1, K=3, I=128, router_std=0.05, bias_range=0.02),
    LayerConfig("one_expert", T=130, H=384, E=1, G=1, Mg=1, K=1, I=256, router_std=0.05),
    LayerConfig("wide", T=300, H=1024, E=32, G=8, Mg=4, K=8, I=384, router_std=0.02, bias_range=0.01),
    # few tokens: the shared expert's down-projection with the combine runs on
    # 16- and 32-row weight-streaming tiles
    LayerConfig("few7", T=7, H=512, E=16, G=4, Mg=2, K=4, I=256, router_std=0.05),
    LayerConfig("few20", T=20, H=512, E=16, G=4, Mg=2, K=4, I=256, router_std=0.05),
    # 256 experts or a multiple: the router logits take the 128 x 256 tiles,
    # here with H split in two (ragged last token tile) and in four (two
    # expert tiles)
    LayerConfig("e256", T=300, H=512, E=256, G=8, Mg=4, K=8, I=128, router_std=0.02, bias_range=0.01),
    LayerConfig("e512", T=128, H=1024, E=512, G=8, Mg=4, K=8, I=128, router_std=0.02, bias_range=0.01),
], ids=lambda c: c.name)
def test_layer_shapes(cfg):
    _layer_case(cfg, torch.float32)


# The kernel instantiations the V3 workloads run, on whole groups at a size
# the oracle checks token by token:
#  * 125 rows per expert: gemm_ws_kernel with 176-row tiles for the gate/up
#    launch (SwiGLU + requant epilogue) and the routed down launch, as at V3
#    prefill (128 rows per expert); groups past 128 rows reach the guarded
#    tail slices of the tile;
#  * 300 rows per expert: gemm_lds2_kernel (256 x 256 tiles) for both
#    launches, as for the hot experts under skew; groups span two row tiles,
#    I = 384 gives three gate/up column tiles.
HEADLINE_CFGS = [
    (LayerConfig("bm176", T=500, H=1024, E=16, G=4, Mg=2, K=4, I=256, router_std=0.02, bias_range=0.01), 176),
    (LayerConfig("lds2", T=1200, H=768, E=16, G=4, Mg=2, K=4, I=384, router_std=0.02, bias_range=0.01), 0),
]


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("cfg,bm", HEADLINE_CFGS, ids=lambda c: getattr(c, "name", str(c)))
def test_layer_headline_tiles(cfg, bm, out_dtype):
    hint = -(-cfg.T * cfg.K // cfg.E)
    assert _ws_tile_rows(hint) == bm
    _, counts, _ = _layer_case(cfg, out_dtype)
    c = host(counts)
    print(f"[tiles] {cfg.name}: rows per expert min {c.min()} mean {c.mean():.0f} max {c.max()}", flush=True)
    if bm:
        assert c.max() > 128, "no group reaches the guarded tail slices of the 176-row tile"
    else:
        assert c.max() > 256, "no group spans two 256-row tiles"


def test_layer_without_shared_expert():
    cfg = LayerConfig("noshared", T=200, H=256, E=16, G=4, Mg=2, K=4, I=128, router_std=0.05)
    _layer_case(cfg, torch.float32, n_shared=0)


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("n_extra", [0, 1, 6, 40])
def test_tiny_layer_serving(out_dtype, n_extra):
    """The decode-serving forward on the tiny layer: no copies (the shared
    expert as a routed group only), one, a few, and more copies than experts."""
    _layer_case(LAYER_CONFIGS["tiny"], out_dtype, serving_extra=n_extra)


@pytest.mark.parametrize("cfg", [
    LayerConfig("ragged", T=77, H=256, E=8, G=2, Mg=1, K=3, I=128, router_std=0.05, bias_range=0.02),
    LayerConfig("one_expert", T=130, H=384, E=1, G=1, Mg=1, K=1, I=256, router_std=0.05),
    LayerConfig("few7", T=7, H=512, E=16, G=4, Mg=2, K=4, I=256, router_std=0.05),
], ids=lambda c: c.name)
def test_layer_shapes_serving(cfg):
    """Serving with 3 extra slots: one expert cut into four, slots left empty
    when an expert has fewer rows than slots (7 tokens)."""
    _layer_case(cfg, torch.float32, serving_extra=3)


def test_layer_serving_without_shared_expert():
    cfg = LayerConfig("noshared", T=200, H=256, E=16, G=4, Mg=2, K=4, I=128, router_std=0.05)
    _layer_case(cfg, torch.float32, n_shared=0, serving_extra=8)


def test_layer_zero_tokens():
    d = _dsmoe()
    cfg = LAYER_CONFIGS["tiny"]
    inp = layer_inputs_host(cfg, 0)
    w13 = dev(inp["w13"], torch.bfloat16)
    w2 = dev(inp["w2"], torch.bfloat16)
    weights = d.quantize_layer_weights(w13[:cfg.E], w2[:cfg.E], dev(inp["router_w"], torch.bfloat16),
                                       w13[cfg.E], w2[cfg.E])
    desc = d.MoEDesc(cfg.H, cfg.I, cfg.E, cfg.G, cfg.Mg, cfg.K, 1)
    x = torch.empty((0, cfg.H), dtype=torch.bfloat16, device="cuda")
    counts = torch.full((cfg.E,), 5, dtype=torch.int32, device="cuda")
    y, counts, _ = d.moe_forward(desc, weights, dev(inp["bias"]), x, counts=counts)
    assert y.shape == (0, cfg.H)
    assert host(counts).sum() == 0


# ---------------------------------------------------------------------------
# DeepSeek-V3 shapes at full size
# ---------------------------------------------------------------------------

# The oracle's codes of the V3-sized expert weights (every V3 workload draws
# the same experts), filled on demand and kept for the session.
_ORACLE_W = {}


def _oracle_weights(cfg, experts):
    from concurrent.futures import ThreadPoolExecutor
    missing = sorted(set(int(e) for e in experts) - set(_ORACLE_W))
    if missing:
        banner(f"oracle: quantising {len(missing)} V3 experts on the host")

    def quant(item):
        e, a, b = item
        return e, oq.quant_w_128x128(a) + oq.quant_w_128x128(b)

    with ThreadPoolExecutor(max_workers=N_CPU) as ex:
        for i in range(0, len(missing), N_CPU):
            batch = []
            for e in missing[i:i + N_CPU]:   # bf16 weights back to the host (same generator)
                a, b = expert_weights_device(cfg, e, "cuda")
                batch.append((e, a.float().cpu().numpy(), b.float().cpu().numpy()))
            for e, w in ex.map(quant, batch):
                _ORACLE_W[e] = w
            print(f"[oracle] {min(i + N_CPU, len(missing))} of {len(missing)} experts quantised", flush=True)
    return _ORACLE_W


def _oracle_tokens(cfg, inp, g, toks, n_per=4):
    """moe_layer on the tokens `toks` (GPU logits, GPU codes of a), in
    parallel chunks of n_per tokens; each token's result depends on that
    token alone.  Returns the chunks' results merged along the token axis."""
    from threadpoolctl import threadpool_limits
    cache = _oracle_weights(cfg, np.unique(g["topk_idx"][toks]).tolist() + [cfg.E])
    T, K, E = cfg.T, cfg.K, cfg.E

    def one(part):
        return ol.moe_layer(inp["x"][part], inp["router_w"], inp["bias"], lambda e: cache[e], cache[E],
                            cfg.G, cfg.Mg, K, logits=g["logits"][part], h_rel_err=lp.H_REL_ERR,
                            a_codes=lp.gpu_a_codes(g, T, K, part, 1, cfg.I))

    parts = [toks[i:i + n_per] for i in range(0, len(toks), n_per)]
    with threadpool_limits(limits=1), concurrent.futures.ThreadPoolExecutor(max_workers=N_CPU) as ex:
        res = list(ex.map(one, parts))
    keys = ("qx", "sx", "logits64", "logits_d", "topk_idx", "gates", "y", "y_d", "qa", "sa", "amb", "lo", "hi",
            "sa_tol", "qa_sh", "sa_sh", "amb_sh", "lo_sh", "hi_sh", "sa_tol_sh")
    return {k: np.concatenate([r[k] for r in res]) for k in keys}


def _v3_weights(d, cfg):
    E, H, I = cfg.E, cfg.H, cfg.I
    q13 = torch.empty((E, 2 * I, H), dtype=torch.uint8, device="cuda")
    s13 = torch.empty((E, 2 * I // 128, H // 128), dtype=torch.float32, device="cuda")
    q2 = torch.empty((E, H, I), dtype=torch.uint8, device="cuda")
    s2 = torch.empty((E, H // 128, I // 128), dtype=torch.float32, device="cuda")
    q13s = torch.empty((2 * I, H), dtype=torch.uint8, device="cuda")
    s13s = torch.empty((2 * I // 128, H // 128), dtype=torch.float32, device="cuda")
    q2s = torch.empty((H, I), dtype=torch.uint8, device="cuda")
    s2s = torch.empty((H // 128, I // 128), dtype=torch.float32, device="cuda")
    for e in range(E + 1):
        a, b = expert_weights_device(cfg, e, "cuda")
        if e < E:
            d.quant_w_128x128(a, q13[e], s13[e])
            d.quant_w_128x128(b, q2[e], s2[e])
        else:
            d.quant_w_128x128(a, q13s, s13s)
            d.quant_w_128x128(b, q2s, s2s)
    return q13, s13, q2, s2, q13s, s13s, q2s, s2s


def _group_checks(cfg, g, inp, offsets, perm, name, row_ranges):
    """Codes of a over whole row ranges of the gate/up launch: each item is
    (label, expert, first row, end row) with expert == E for the shared
    expert (rows T*K + t)."""
    T, K, E = cfg.T, cfg.K, cfg.E
    cache = _oracle_weights(cfg, [e for _, e, _, _ in row_ranges])
    for label, e, r0, r1 in row_ranges:
        if e == E:
            toks = np.arange(r0, r1)
            rows = T * K + toks
        else:
            rows = np.arange(offsets[e] + r0, offsets[e] + r1)
            toks = perm[rows]
        banner(f"layer {name}: codes of a, {label} (expert {e}, {len(rows)} rows)")
        lp.check_group_codes(g, inp["x"], rows, toks, cache[e][0], cache[e][1], f"{name} {label}")


def _v3_case(name, n_sample, out_dtype=torch.bfloat16, serving_extra=None, group_ranges=None):
    d = _dsmoe()
    cfg = LAYER_CONFIGS[name]
    E, H, I, T, K = cfg.E, cfg.H, cfg.I, cfg.T, cfg.K
    banner(f"layer {name} full size: quantising {E + 1} experts")
    inp = layer_inputs_host(cfg, 0, with_weights=False)
    w = _v3_weights(d, cfg)
    weights = d.MoEWeights(*w, dev(inp["router_w"], torch.bfloat16))
    desc = d.MoEDesc(H, I, E, cfg.G, cfg.Mg, K, 1)
    banner(f"layer {name} full size: forward T={T}")
    x_dev = dev(inp["x"], torch.bfloat16)
    y, counts, dbg = d.moe_forward(desc, weights, dev(inp["bias"]), x_dev, out_dtype=out_dtype, debug=True)
    g = _gpu(dbg, counts)
    del dbg
    _check_perm_valid(g, T, K, E)
    _, (_, offsets, perm, _) = lp.check_routing_all(g, inp["bias"], cfg.G, cfg.Mg, K, E, name)

    rng = np.random.default_rng(3)
    if n_sample >= T:
        toks = np.arange(T)
    else:
        toks = np.unique(np.concatenate([[0, T - 1], rng.choice(T, size=n_sample - 2, replace=False)]))
    banner(f"layer {name} full size: oracle on {len(toks)} tokens")
    want = _oracle_tokens(cfg, inp, g, toks)
    # spot-check the GPU's weight codes against the oracle's on two experts
    for e in sorted(set(g["topk_idx"][toks].reshape(-1).tolist()))[:2]:
        assert np.array_equal(host(w[0][e]), _ORACLE_W[e][0])
        assert np.array_equal(host(w[1][e]).view(np.uint32), _ORACLE_W[e][1].view(np.uint32))
    yh = host(y)
    lp.check_tokens(g, yh, want, toks, T, K, 1, DT[out_dtype], f"{name} sampled")
    if group_ranges is not None:
        _group_checks(cfg, g, inp, offsets, perm, name, group_ranges(g["counts"]))
    if serving_extra is not None:
        banner(f"layer {name} serving: {serving_extra} extra slots")
        y2, c2, dbg2, _ = _serving(d, desc, weights, counts, serving_extra, dev(inp["bias"]), x_dev, out_dtype)
        g2 = _gpu(dbg2, c2)
        for k in ("counts", "topk_idx", "perm", "inv"):
            assert np.array_equal(g2[k], g[k]), f"serving {k} differs from the plain forward's"
        want2 = _oracle_tokens(cfg, inp, g2, toks)
        lp.check_tokens(g2, host(y2), want2, toks, T, K, 1, DT[out_dtype], f"{name} serving sampled")
    return g


def _prefill_groups(counts):
    """The largest and the smallest routed group whole (176-row tiles; the
    largest passes 128 rows, into the guarded tail slices), the shared
    expert's first two tiles and its ragged last one."""
    E = len(counts)
    T = LAYER_CONFIGS["v3_prefill"].T
    e_big = int(np.argmax(counts))
    nz = np.nonzero(counts)[0]
    e_small = int(nz[np.argmin(counts[nz])])
    assert counts[e_big] > 128
    return [("largest group", e_big, 0, int(counts[e_big])),
            ("smallest group", e_small, 0, int(counts[e_small])),
            ("shared tiles 0-1", E, 0, 352), ("shared last tile", E, (T // 176) * 176, T)]


def _skew_groups(counts):
    """The hottest expert's first two 256-row tiles and its ragged last tile,
    a tail expert, and the shared expert's first two tiles."""
    order = np.argsort(-counts, kind="stable")
    hot = int(order[0])
    c = int(counts[hot])
    tail = int(order[np.nonzero(counts[order] > 0)[0][-1]])
    last0 = (c - 1) // 256 * 256
    return [("hottest tiles 0-1", hot, 0, 512), ("hottest last tile", hot, last0, c),
            ("tail group", tail, 0, int(counts[tail])), ("shared tiles 0-1", len(counts), 0, 512)]


def test_v3_prefill_full_size():
    _v3_case("v3_prefill", n_sample=64, group_ranges=_prefill_groups)


def test_v3_decode_full_size():
    # T = 64: every token, every code
    _v3_case("v3_decode", n_sample=64, out_dtype=torch.float32)


def test_v3_prefill_serving_full_size():
    """The serving forward at V3 prefill size (T = 4096, groups of ~128 rows
    split over 32 extra slots, the shared expert's 4096 rows as one group of
    the routed launches)."""
    _v3_case("v3_prefill", n_sample=32, serving_extra=32)


def test_v3_decode_serving_full_size():
    """The decode-serving forward at V3 decode size with 64 copies of hot
    experts (the inference paragraph's 256 + 64) planned from this step's loads."""
    _v3_case("v3_decode", n_sample=64, out_dtype=torch.float32, serving_extra=64)


def test_v3_skew_full_size():
    # Zipf(1.1) expert popularity: the hot experts' groups (thousands of rows)
    # run on 256 x 256 tiles, the tail on the same launch's nearly empty tiles
    g = _v3_case("v3_skew", n_sample=64, group_ranges=_skew_groups)
    assert g["counts"].max() > 8 * g["counts"].mean()
