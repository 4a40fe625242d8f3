"""GPU parity of dsmoe_moe_forward against the oracle's layer.

* qx / sx (the 1x128 codes of x): bit-exact.
* logits: |gpu - oracle| <= 2e-5 * (|x| . |Wr|^T).  The GPU accumulates
  bf16 products (exact in FP32) in FP32 over H/32 MFMA steps; the bound is
  the FP32 summation error of that depth (about (H/32 + 5) * 2^-24 relative
  to the absolute sum, i.e. 1.4e-5 at H = 7168), rounded up.
* routing: the oracle routes on its own float64 logits rounded to float32.
  Tokens whose choice is unique under both logit sets must match exactly;
  a token may only differ where its keys are tied within the logit bound,
  and then the GPU's choice must be one of the valid ones.
* y on tokens with identical routing: max |gpu - oracle| / y_d <= 2e-3
  (float32 y) or 1e-2 (bf16 y), y_d = sum_k gate_k |a_hat| . |w2_hat|^T plus
  the shared expert's term.
"""

import concurrent.futures

import numpy as np
import pytest
import torch

from dsmoe_inputs import LAYER_CONFIGS, LayerConfig, expert_weights_device, layer_inputs_host
from gpu_util import assert_normalised_close, banner, dev, host
from oracle import layer as ol
from oracle import quant as oq
from oracle import route as orr

pytestmark = pytest.mark.gpu

Y_TOL = {torch.float32: 2e-3, torch.bfloat16: 1e-2}
LOGIT_TOL = 2e-5
# Bound on the GPU's error in h = x W13^T relative to |x_hat| . |w13_hat|:
# a chunk's 128 products summed in FP32 (<= 128 roundings), the scale
# product and the FP32 accumulation over up to H/128 = 56 chunks:
# (128 + 56 + 2) * 2^-24 = 1.1e-5, rounded up.
H_REL_ERR = 2e-5


def _dsmoe():
    import fp8_block_scaled_dsmoe_amd as d
    return d


def _check_routing(cfg, gpu_idx, want, keys64, logit_bound):
    """Return the mask of tokens whose routing matches exactly; assert that
    every other token is a near-tie where the GPU's choice is valid."""
    same = np.all(gpu_idx == want["topk_idx"], axis=1)
    per = cfg.E // cfg.G
    for t in np.nonzero(~same)[0]:
        g_sel = gpu_idx[t]
        assert len(set(g_sel.tolist())) == cfg.K, f"token {t}: repeated expert"
        assert len(set((g_sel // per).tolist())) <= cfg.Mg, f"token {t}: too many groups"
        # keys move by at most slope(1/4) * logit bound (+ rounding)
        eps = 0.25 * logit_bound[t] + 2e-7
        k_gpu = np.sort(keys64[t, g_sel])[::-1]
        k_or = np.sort(keys64[t, want["topk_idx"][t]])[::-1]
        assert np.all(np.abs(k_gpu - k_or) <= 4 * eps), \
            f"token {t}: GPU routing {g_sel.tolist()} differs from the oracle's " \
            f"{want['topk_idx'][t].tolist()} beyond a near-tie (keys {k_gpu} vs {k_or})"
    n_diff = int((~same).sum())
    print(f"[parity] routing: {n_diff} of {len(same)} tokens differ (near-ties)", flush=True)
    assert n_diff <= max(2, len(same) // 500)
    return same


def _check_perm_valid(gpu, T, K, E):
    idx = gpu["topk_idx"]
    counts = np.bincount(idx.reshape(-1), minlength=E)
    assert np.array_equal(gpu["counts"], counts)
    assert np.array_equal(gpu["offsets"], np.concatenate([[0], np.cumsum(counts)]))
    perm, inv, off = gpu["perm"], gpu["inv"], gpu["offsets"]
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
    y, c = d.moe_forward_serving(desc, slot_w, slot_first, slot_expert, bias, x, out_dtype=out_dtype)
    return y, c, slot_first


def _layer_case(cfg: LayerConfig, out_dtype, n_shared=1, seed=0, serving_extra=None):
    d = _dsmoe()
    inp = layer_inputs_host(cfg, seed)
    banner(f"layer {cfg.name} T={cfg.T} H={cfg.H} E={cfg.E} K={cfg.K} shared={n_shared} {out_dtype}")
    x = dev(inp["x"], torch.bfloat16)
    wr = dev(inp["router_w"], torch.bfloat16)
    w13 = dev(inp["w13"], torch.bfloat16)
    w2 = dev(inp["w2"], torch.bfloat16)
    weights = d.quantize_layer_weights(w13[:cfg.E], w2[:cfg.E], wr,
                                       w13[cfg.E] if n_shared else None, w2[cfg.E] if n_shared else None)
    desc = d.MoEDesc(cfg.H, cfg.I, cfg.E, cfg.G, cfg.Mg, cfg.K, n_shared)
    y, counts, dbg = d.moe_forward(desc, weights, dev(inp["bias"]), x, out_dtype=out_dtype, debug=True)

    q13, s13 = oq.quant_w_128x128(inp["w13"])
    q2, s2 = oq.quant_w_128x128(inp["w2"])
    assert np.array_equal(host(weights.w13), q13[:cfg.E])
    assert np.array_equal(host(weights.s2).view(np.uint32), s2[:cfg.E].view(np.uint32))
    get = lambda e: (q13[e], s13[e], q2[e], s2[e])
    if n_shared:
        shared = get(cfg.E)
    else:
        zero13 = np.zeros_like(q13[0]); zero2 = np.zeros_like(q2[0])
        shared = (zero13, np.ones_like(s13[0]), zero2, np.ones_like(s2[0]))
    want = ol.moe_layer(inp["x"], inp["router_w"], inp["bias"], get, shared, cfg.G, cfg.Mg, cfg.K,
                        h_rel_err=H_REL_ERR)
    print(f"[parity] {want['n_ambiguous']} FP8 codes of a are decided within the error of h", flush=True)

    g = {k: host(v) for k, v in dbg.items()}
    g["counts"] = host(counts)
    assert np.array_equal(g["qx"], want["qx"])
    assert np.array_equal(g["sx"].view(np.uint32), want["sx"].view(np.uint32))
    assert_normalised_close(g["logits"], want["logits64"], want["logits_d"], LOGIT_TOL, "logits")
    keys64 = orr.keys(orr.affinity(want["logits64"].astype(np.float32)), inp["bias"]).astype(np.float64)
    bound = LOGIT_TOL * want["logits_d"].max(axis=1)
    same = _check_routing(cfg, g["topk_idx"], want, keys64, bound)
    _check_perm_valid(g, cfg.T, cfg.K, cfg.E)
    if same.all():
        assert np.array_equal(g["counts"], want["counts"])
        assert np.array_equal(g["perm"], want["perm"])
        assert np.array_equal(g["inv"], want["inv"])
    assert np.abs(g["gates"][same] - want["gates"][same]).max(initial=0) <= 1e-6
    yh = host(y)
    assert_normalised_close(yh[same], want["y"][same], want["y_d"][same], Y_TOL[out_dtype],
                            f"y {cfg.name} {out_dtype}", slack=want["y_slack"][same])
    if serving_extra is not None:
        # the decode-serving forward: slots planned from this step's loads, the
        # shared expert as one more routed group; same routing, same bar
        banner(f"layer {cfg.name} serving: {serving_extra} extra slots")
        y2, c2, slot_first = _serving(d, desc, weights, counts, serving_extra, dev(inp["bias"]), x, out_dtype)
        assert np.array_equal(host(c2), g["counts"])
        n_rep = np.diff(host(slot_first))
        print(f"[serving] slots per expert: max {n_rep.max()}, max rows per slot "
              f"{(g['counts'] / n_rep).max():.1f} (was {g['counts'].max()})", flush=True)
        assert_normalised_close(host(y2)[same], want["y"][same], want["y_d"][same], Y_TOL[out_dtype],
                                f"y serving {cfg.name} {out_dtype}", slack=want["y_slack"][same])
    return y, counts


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_tiny_layer(out_dtype):
    _layer_case(LAYER_CONFIGS["tiny"], out_dtype)


def test_tiny_layer_deterministic():
    cfg = LAYER_CONFIGS["tiny"]
    y1, c1 = _layer_case(cfg, torch.float32)
    y2, c2 = _layer_case(cfg, torch.float32)
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
], ids=lambda c: c.name)
def test_layer_shapes(cfg):
    _layer_case(cfg, torch.float32)


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
# DeepSeek-V3 shapes at full size, checked on sampled tokens
# ---------------------------------------------------------------------------

def _v3_case(name: str, n_sample: int, out_dtype=torch.bfloat16, serving_extra=None):
    d = _dsmoe()
    cfg = LAYER_CONFIGS[name]
    E, H, I = cfg.E, cfg.H, cfg.I
    banner(f"layer {name} full size: quantising {E + 1} experts")
    inp = layer_inputs_host(cfg, 0, with_weights=False)
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
    wr = dev(inp["router_w"], torch.bfloat16)
    weights = d.MoEWeights(q13, s13, q2, s2, q13s, s13s, q2s, s2s, wr)
    desc = d.MoEDesc(H, I, E, cfg.G, cfg.Mg, cfg.K, 1)
    banner(f"layer {name} full size: forward T={cfg.T}")
    y, counts, dbg = d.moe_forward(desc, weights, dev(inp["bias"]), dev(inp["x"], torch.bfloat16),
                                   out_dtype=out_dtype, debug=True)
    torch.cuda.synchronize()
    g = {k: host(v) for k, v in dbg.items()}
    g["counts"] = host(counts)
    _check_perm_valid(g, cfg.T, cfg.K, E)

    rng = np.random.default_rng(3)
    toks = np.unique(np.concatenate([[0, cfg.T - 1], rng.choice(cfg.T, size=n_sample - 2, replace=False)]))
    xs = inp["x"][toks]
    z64, _ = ol.router_logits(xs, inp["router_w"])
    r_or = orr.route(z64.astype(np.float32), inp["bias"], cfg.G, cfg.Mg, cfg.K)
    needed = sorted(set(r_or["topk_idx"].reshape(-1).tolist()) | {E})
    banner(f"layer {name} full size: oracle on {len(toks)} tokens, {len(needed)} experts")

    host_w = {}
    for e in needed:   # bf16 weights back to host (same generator as above)
        a, b = expert_weights_device(cfg, e, "cuda")
        host_w[e] = (a.float().cpu().numpy(), b.float().cpu().numpy())

    def quantise(e):
        q13_o, s13_o = oq.quant_w_128x128(host_w[e][0])
        q2_o, s2_o = oq.quant_w_128x128(host_w[e][1])
        return e, (q13_o, s13_o, q2_o, s2_o)

    with concurrent.futures.ThreadPoolExecutor(max_workers=8) as ex:
        cache = dict(ex.map(quantise, needed))
    # spot-check the GPU's weight codes against the oracle's on two experts
    for e in needed[:2]:
        src = (q13s, s13s) if e == E else (q13[e], s13[e])
        assert np.array_equal(host(src[0]), cache[e][0])
        assert np.array_equal(host(src[1]).view(np.uint32), cache[e][1].view(np.uint32))
    want = ol.moe_layer(xs, inp["router_w"], inp["bias"], lambda e: cache[e], cache[E],
                        cfg.G, cfg.Mg, cfg.K, h_rel_err=H_REL_ERR)
    assert np.array_equal(g["qx"][toks], want["qx"])
    assert np.array_equal(g["sx"][toks].view(np.uint32), want["sx"].view(np.uint32))
    assert_normalised_close(g["logits"][toks], want["logits64"], want["logits_d"], LOGIT_TOL,
                            f"logits {name}")
    keys64 = orr.keys(orr.affinity(want["logits64"].astype(np.float32)), inp["bias"]).astype(np.float64)
    sub = LayerConfig("s", T=len(toks), H=H, E=E, G=cfg.G, Mg=cfg.Mg, K=cfg.K, I=I, router_std=0)
    same = _check_routing(sub, g["topk_idx"][toks], want, keys64,
                          LOGIT_TOL * want["logits_d"].max(axis=1))
    yh = host(y)[toks]
    assert_normalised_close(yh[same], want["y"][same], want["y_d"][same], Y_TOL[out_dtype],
                            f"y {name} sampled", slack=want["y_slack"][same])
    if serving_extra is not None:
        banner(f"layer {name} serving: {serving_extra} extra slots")
        y2, c2, _ = _serving(d, desc, weights, counts, serving_extra, dev(inp["bias"]),
                             dev(inp["x"], torch.bfloat16), out_dtype)
        assert np.array_equal(host(c2), g["counts"])
        assert_normalised_close(host(y2)[toks][same], want["y"][same], want["y_d"][same], Y_TOL[out_dtype],
                                f"y serving {name} sampled", slack=want["y_slack"][same])
    return g


def test_v3_prefill_full_size_sampled():
    _v3_case("v3_prefill", n_sample=4)


def test_v3_decode_full_size_sampled():
    _v3_case("v3_decode", n_sample=4, out_dtype=torch.float32)


def test_v3_prefill_serving_full_size_sampled():
    """The serving forward at V3 prefill size (T = 4096, groups of ~128 rows
    split over 32 extra slots, the shared expert's 4096 rows as one group of
    the routed launches)."""
    _v3_case("v3_prefill", n_sample=4, serving_extra=32)


def test_v3_decode_serving_full_size_sampled():
    """The decode-serving forward at V3 decode size with 64 copies of hot
    experts (the inference paragraph's 256 + 64) planned from this step's loads."""
    _v3_case("v3_decode", n_sample=4, out_dtype=torch.float32, serving_extra=64)


def test_v3_skew_full_size_sampled():
    # Zipf(1.1) expert popularity: the hot experts' groups (thousands of rows)
    # run on 256 x 256 tiles, the tail on weight-streaming tiles
    g = _v3_case("v3_skew", n_sample=4)
    assert g["counts"].max() > 8 * g["counts"].mean()
