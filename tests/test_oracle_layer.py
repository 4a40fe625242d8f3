"""Pins of the oracle's expert FFN and layer forward.

* a scalar re-derivation of one expert FFN from decode_scalar/encode_scalar,
  math.exp and explicit loops (pins the gate/up row layout, silu, the
  float32 rounding of a and its 1x128 requantisation);
* identical routed experts: gates sum to 1, so y = FFN_shared(x) + FFN(x) for
  any routing (pins permute, gate normalisation and combine);
* one expert, top-1: y = FFN_shared(x) + FFN_0(x);
* zero input gives exactly zero output.
"""

import math

import numpy as np
import pytest

from oracle import e4m3, layer, quant
from dsmoe_inputs import LayerConfig, layer_inputs_host, normal_bf16


def _scalar_ffn_row(x_row, w13, w2):
    """One token through one expert, written with scalar primitives only."""
    H = x_row.shape[0]
    I2 = w13.shape[0]
    I = I2 // 2

    def quant_row(v):
        codes, scales = [], []
        for j in range(0, len(v), 128):
            tile = [float(np.float32(t)) for t in v[j:j + 128]]
            amax = max(abs(t) for t in tile)
            s = float(np.float32(np.float32(amax) / np.float32(448.0))) if amax else 1.0
            for t in tile:
                codes.append(e4m3.encode_scalar(float(np.float32(np.float32(t) / np.float32(s)))))
            scales.append(s)
        return codes, scales

    def quant_block(w):
        n, k = w.shape
        q = np.zeros((n, k), np.uint8)
        s = np.zeros((n // 128, k // 128))
        for bi in range(n // 128):
            for bj in range(k // 128):
                blk = w[bi * 128:(bi + 1) * 128, bj * 128:(bj + 1) * 128]
                amax = float(np.max(np.abs(blk)))
                sc = float(np.float32(np.float32(amax) / np.float32(448.0))) if amax else 1.0
                s[bi, bj] = sc
                for i in range(128):
                    for j in range(128):
                        q[bi * 128 + i, bj * 128 + j] = e4m3.encode_scalar(
                            float(np.float32(np.float32(blk[i, j]) / np.float32(sc))))
        return q, s

    def dot_row(codes, scales, q, s, n):
        total = 0.0
        for c in range(len(scales)):
            part = 0.0
            for k in range(c * 128, (c + 1) * 128):
                part += e4m3.decode_scalar(codes[k]) * e4m3.decode_scalar(q[n, k])
            total += scales[c] * s[n // 128, c] * part
        return total

    qx, sx = quant_row(x_row)
    q13, s13 = quant_block(w13)
    q2, s2 = quant_block(w2)
    h = [dot_row(qx, sx, q13, s13, n) for n in range(I2)]
    a = []
    for j in range(I):
        g, u = h[j], h[I + j]
        a.append(float(np.float32(g / (1.0 + math.exp(-g)) * u)))
    qa, sa = quant_row(a)
    return np.array([dot_row(qa, sa, q2, s2, n) for n in range(H)])


def test_expert_ffn_matches_scalar_derivation():
    H, I = 256, 128
    x = normal_bf16("ffn_x", (2, H), 1.0, seed=4)
    w13 = normal_bf16("ffn_w13", (2 * I, H), 0.05, seed=4)
    w2 = normal_bf16("ffn_w2", (H, I), 0.05, seed=4)
    qx, sx = quant.quant_act_1x128(x)
    q13, s13 = quant.quant_w_128x128(w13)
    q2, s2 = quant.quant_w_128x128(w2)
    o, d = layer.expert_ffn(qx, sx, q13, s13, q2, s2)
    for r in range(2):
        want = _scalar_ffn_row(x[r], w13, w2)
        assert np.allclose(o[r], want, rtol=1e-12, atol=1e-12 * np.max(d[r]))
    assert np.all(np.abs(o) <= d * (1 + 1e-12))


def _quantised_experts(w13, w2):
    q13, s13 = quant.quant_w_128x128(w13)
    q2, s2 = quant.quant_w_128x128(w2)
    return q13, s13, q2, s2


def _small_cfg(E, G, Mg, K):
    return LayerConfig("t", T=48, H=256, E=E, G=G, Mg=Mg, K=K, I=128, router_std=0.05)


def test_identical_experts_give_dense_ffn():
    cfg = _small_cfg(8, 4, 2, 3)
    d = layer_inputs_host(cfg, seed=9)
    d["bias"] = np.linspace(-0.05, 0.05, cfg.E).astype(np.float32)
    q13, s13, q2, s2 = _quantised_experts(d["w13"], d["w2"])
    same = (q13[0], s13[0], q2[0], s2[0])
    shared = (q13[cfg.E], s13[cfg.E], q2[cfg.E], s2[cfg.E])
    out = layer.moe_layer(d["x"], d["router_w"], d["bias"], lambda e: same, shared,
                          cfg.G, cfg.Mg, cfg.K)
    qx, sx = quant.quant_act_1x128(d["x"])
    o_sh, _ = layer.expert_ffn(qx, sx, *shared)
    o_0, _ = layer.expert_ffn(qx, sx, *same)
    assert np.allclose(out["y"], o_sh + o_0, rtol=1e-12, atol=1e-12 * np.max(np.abs(o_0)))
    # routing really spread the tokens over several experts
    assert np.count_nonzero(out["counts"]) >= 4


def test_single_expert_top1_is_two_dense_ffns():
    cfg = _small_cfg(1, 1, 1, 1)
    d = layer_inputs_host(cfg, seed=2)
    q13, s13, q2, s2 = _quantised_experts(d["w13"], d["w2"])
    get = lambda e: (q13[e], s13[e], q2[e], s2[e])
    out = layer.moe_layer(d["x"], d["router_w"], d["bias"], get, get(1), 1, 1, 1)
    qx, sx = quant.quant_act_1x128(d["x"])
    want = layer.expert_ffn(qx, sx, *get(1))[0] + layer.expert_ffn(qx, sx, *get(0))[0]
    assert np.array_equal(out["gates"], np.ones((cfg.T, 1)))
    assert np.allclose(out["y"], want, rtol=1e-13, atol=0)


def test_zero_input_gives_zero_output():
    cfg = _small_cfg(8, 2, 1, 2)
    d = layer_inputs_host(cfg, seed=3)
    x = np.zeros_like(d["x"])
    q13, s13, q2, s2 = _quantised_experts(d["w13"], d["w2"])
    get = lambda e: (q13[e], s13[e], q2[e], s2[e])
    out = layer.moe_layer(x, d["router_w"], d["bias"], get, get(cfg.E), cfg.G, cfg.Mg, cfg.K)
    assert np.all(out["y"] == 0)
    assert out["counts"].sum() == cfg.T * cfg.K


def test_requant_ambiguity_flags_codes_at_midpoints_only():
    # one 128-wide tile with amax 448 (scale 1): 17 sits on the 16/18 midpoint,
    # 16 is a code value, 17.5 is half a step from both of its midpoints
    a = np.zeros((1, 128), np.float32)
    a[0, :4] = [448.0, 17.0, 16.0, 17.5]
    qa, sa = quant.quant_act_1x128(a)
    assert sa[0, 0] == 1.0
    h = np.zeros((1, 256))
    h_d = np.zeros((1, 256))
    amb, lo, hi, sa_tol = layer.requant_ambiguity(h, h_d, a, qa, sa, 0.0)
    assert amb.sum() == 1 and amb[0, 1]
    assert (lo[0, 1], hi[0, 1]) == (16.0, 18.0)
    assert (lo[0, 2], hi[0, 2]) == (16.0, 16.0) and (lo[0, 3], hi[0, 3]) == (18.0, 18.0)
    assert (lo[0, 0], hi[0, 0]) == (448.0, 448.0) and np.all(lo[0, 4:] == 0) and np.all(hi[0, 4:] == 0)
    # with no error in h the scale may move only by the float32 evaluation of
    # a (8 ulps of the amax, over 448) and one ulp of the division
    assert sa_tol[0, 0] == 8 * 2.0 ** -24 + 2.0 ** -23
    # a large error bound makes every element ambiguous, zeros included, over
    # the whole code range
    amb_all, lo_all, hi_all, _ = layer.requant_ambiguity(h + 1.0, np.ones((1, 256)) * 1e3, a, qa, sa, 1.0)
    assert amb_all.sum() == 128 and np.all(lo_all == -448.0) and np.all(hi_all == 448.0)


@pytest.mark.parametrize("rel", [2e-5, 5e-4])
def test_requant_ambiguity_covers_perturbed_implementations(rel):
    # An implementation whose h is off by up to rel * h_d (here every element
    # pushed almost to the bound with a random sign) and which evaluates silu(g) * u
    # in float32 must land on a code inside the valid range everywhere (the
    # oracle's code wherever the range is one code), and within sa_tol on the
    # scales.  The larger error moves small values by several codes.
    H, I, n = 512, 256, 400
    x = normal_bf16("amb_x", (n, H), 1.0, seed=6)
    w13 = normal_bf16("amb_w13", (2 * I, H), 0.02, seed=6)
    qx, sx = quant.quant_act_1x128(x)
    q13, s13 = quant.quant_w_128x128(w13)
    h, a32, qa, sa = layer.expert_gate_up(qx, sx, q13, s13)
    from oracle.gemm import gemm_normaliser
    h_d = gemm_normaliser(qx, sx, q13, s13)
    amb, lo, hi, sa_tol = layer.requant_ambiguity(h, h_d, a32, qa, sa, rel)
    # (0.999: room for the float32 rounding of the perturbed h itself)
    sign = np.where(np.random.default_rng(1).random(h.shape) < 0.5, -1.0, 1.0)
    hp = (h + sign * 0.999 * rel * h_d).astype(np.float32)
    g, u = hp[:, :I], hp[:, I:]
    with np.errstate(over="ignore"):
        ap = (g / (np.float32(1) + np.exp(-g)) * u).astype(np.float32)
    qp, sp = quant.quant_act_1x128(ap)
    vp = e4m3.decode(qp)
    differ = vp != e4m3.decode(qa)
    assert differ.sum() > 0, "the perturbation should move some codes"
    assert np.all((vp >= lo) & (vp <= hi)), "a code moved outside its valid range"
    assert not np.any(differ & ~amb), "a code moved that is not flagged"
    assert np.all(np.abs(sp.astype(np.float64) - sa) <= sa_tol)
    # the bound is relative to |x_hat| . |w13_hat| (h itself cancels), so it
    # flags more codes than move, but at the FP32 bound still a small share
    if rel < 1e-4:
        assert amb.mean() < 0.1


def test_router_logits_one_hot_rows_pick_router_columns():
    # x rows that are -2 times a unit vector e_h give z[t][e] = -2 Wr[e][h]
    # exactly, and normaliser 2 |Wr[e][h]|; a transposed operand or a dropped
    # absolute value fails this.
    E, H = 6, 256
    wr = normal_bf16("pin_wr", (E, H), 0.3, seed=1)
    hs = np.array([0, 5, 127, 128, 255])
    x = np.zeros((len(hs), H), np.float32)
    x[np.arange(len(hs)), hs] = -2.0
    z, dz = layer.router_logits(x, wr)
    assert z.shape == (len(hs), E)
    assert np.array_equal(z, -2.0 * wr[:, hs].T.astype(np.float64))
    assert np.array_equal(dz, 2.0 * np.abs(wr[:, hs].T).astype(np.float64))
