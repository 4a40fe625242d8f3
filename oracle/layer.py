"""Expert SwiGLU FFN on FP8 inputs and the DeepSeekMoE layer forward.

Sources:
* V3 notes §2: the MoE layer has one shared expert that every token passes
  through plus 256 routed experts of intermediate size 2048, 8 chosen per
  token; the layer output sums the shared expert's output and the routed
  experts' outputs weighted by their gates (the equation itself was lost from
  the page; only "just the 8 top-K gates are non-zero" survives).
* V3 notes §6: the Linear GEMMs run with FP8 inputs and produce BF16/FP32
  outputs; the activation between the two projections is quantised again as
  the down-projection's FP8 input, per 1x128 tile (§6.1).
* infra answer (memory paragraph): SwiGLU is the expert activation (named as
  a recomputation target).

Readings taken where the pages are silent:
* W13 of an expert is [2I][H]: rows 0..I-1 are the gate projection, rows
  I..2I-1 the up projection; a = silu(gate) * up with silu(v) = v/(1+e^-v);
* a is evaluated in float64, rounded once to float32, then 1x128-quantised;
* the shared expert has the same intermediate size I and gate 1;
* the router is not quantised: logits are bf16 x times bf16 router weights,
  evaluated here in float64 (the GPU accumulates in FP32);
* no residual add: the layer returns the FFN output only;
* every (token, expert) pair is computed (no capacity limit, no dropping).
"""

import numpy as np

from .e4m3 import decode
from .gemm import block_scaled_gemm, dequant_w, gemm_normaliser
from .quant import quant_act_1x128
from .route import permute, route

_MAGS = decode(np.arange(127, dtype=np.uint8))       # the 127 non-negative finite magnitudes


def requant_slack(h, h_d, a32, qa, sa, q2, s2, h_rel_err):
    """Bound on how far a valid down-projection output may sit from this one
    because of FP8 codes of a that are decided within the error of h.

    The intermediate a is quantised from values computed in float32 (the
    recipe promotes GEMM partial sums to FP32), so an implementation whose h
    differs from the exact h by up to h_rel_err * |x_hat| . |w13_hat| may
    round an element of a/s that sits that close to a rounding midpoint to
    the neighbouring code; both codes are correct.  For every such element
    the output may move by s * step * |w2_hat|.  Returns (slack float64
    [n][H], number of ambiguous codes).
    """
    inter = h.shape[1] // 2
    g, u = h[:, :inter], h[:, inter:]
    dg, du = h_rel_err * h_d[:, :inter], h_rel_err * h_d[:, inter:]
    with np.errstate(over="ignore"):
        sig = 1.0 / (1.0 + np.exp(-g))
    silu = g * sig
    dsilu = np.abs(sig * (1.0 + g * (1.0 - sig)))
    # first-order error of silu(g) * u, plus float32 evaluation (a few ulps)
    da = dsilu * dg * np.abs(u) + np.abs(silu) * du + dg * du + 8 * 2.0 ** -24 * np.abs(a32)
    n, cols = a32.shape
    s = np.repeat(sa.astype(np.float64), 128, axis=1)
    amax = np.repeat(np.max(np.abs(a32.reshape(n, cols // 128, 128)), axis=2).astype(np.float64), 128, axis=1)
    da_tile = np.repeat(np.max(da.reshape(n, cols // 128, 128), axis=2), 128, axis=1)
    v = np.abs(a32.astype(np.float64)) / s
    # the scale itself may move with the tile's amax
    dv = da / s + v * np.where(amax > 0, da_tile / np.where(amax > 0, amax, 1.0), 0.0)
    c = (qa & 0x7F).astype(np.int64)
    lo_mid = np.where(c > 0, (_MAGS[np.maximum(c - 1, 0)] + _MAGS[c]) / 2, -np.inf)
    hi_mid = np.where(c < 126, (_MAGS[np.minimum(c + 1, 126)] + _MAGS[c]) / 2, np.inf)
    step = np.maximum(np.where(c < 126, _MAGS[np.minimum(c + 1, 126)] - _MAGS[c], 0.0),
                      np.where(c > 0, _MAGS[c] - _MAGS[np.maximum(c - 1, 0)], 0.0))
    amb = (np.abs(v - lo_mid) <= dv) | (np.abs(hi_mid - v) <= dv)
    weight = np.where(amb, s * step, 0.0)
    slack = weight @ np.abs(dequant_w(q2, s2)).T
    return slack, int(amb.sum())


def expert_ffn(qx, sx, q13, s13, q2, s2, h_rel_err=None):
    """One expert on quantised input rows.

    qx uint8 [n][H], sx f32 [n][H/128]; q13 uint8 [2I][H], s13 f32
    [2I/128][H/128]; q2 uint8 [H][I], s2 f32 [H/128][I/128].
    Returns (o float64 [n][H], d float64 [n][H]) where d is the down
    projection's |a_hat| x |w2_hat| normaliser; with h_rel_err given, also
    (slack [n][H], ambiguous code count) from requant_slack.
    """
    inter = q13.shape[0] // 2
    h = block_scaled_gemm(qx, sx, q13, s13)                  # [n][2I]
    gate, up = h[:, :inter], h[:, inter:]
    with np.errstate(over="ignore"):
        a = gate / (1.0 + np.exp(-gate)) * up
    a32 = a.astype(np.float32)
    qa, sa = quant_act_1x128(a32)
    o = block_scaled_gemm(qa, sa, q2, s2)
    d = gemm_normaliser(qa, sa, q2, s2)
    if h_rel_err is None:
        return o, d
    slack, n_amb = requant_slack(h, gemm_normaliser(qx, sx, q13, s13), a32, qa, sa, q2, s2, h_rel_err)
    return o, d, slack, n_amb


def router_logits(x, router_w):
    """z = x . Wr^T in float64, with its normaliser |x| . |Wr|^T."""
    x64 = np.asarray(x, np.float64)
    w64 = np.asarray(router_w, np.float64)
    return x64 @ w64.T, np.abs(x64) @ np.abs(w64).T


def moe_layer(x, router_w, bias, get_expert, shared, n_groups, groups_kept, top_k,
              logits=None, h_rel_err=None):
    """DeepSeekMoE layer forward for the rows of x.

    x           float32 [T][H] holding bf16 values
    router_w    float32 [E][H] holding bf16 values
    bias        float32 [E]
    get_expert  callable e -> (q13, s13, q2, s2) for routed expert e
    shared      (q13, s13, q2, s2) of the shared expert
    logits      optional float32 [T][E]; when given, routing uses them instead
                of the oracle's own float64 logits rounded to float32
    h_rel_err   optional: also return y_slack and n_ambiguous (requant_slack
                summed over the experts with their gates)

    Returns a dict: qx, sx, logits64, logits_d, topk_idx, gates, counts,
    offsets, perm, inv, y (float64 [T][H]) and y_d (its normaliser).
    """
    x = np.asarray(x, np.float32)
    t, h = x.shape
    n_experts = np.asarray(router_w).shape[0]
    qx, sx = quant_act_1x128(x)
    z64, zd = router_logits(x, router_w)
    z32 = z64.astype(np.float32) if logits is None else np.asarray(logits, np.float32)
    r = route(z32, bias, n_groups, groups_kept, top_k)
    counts, offsets, perm, inv = permute(r["topk_idx"], n_experts)

    res = expert_ffn(qx, sx, *shared, h_rel_err=h_rel_err)    # shared expert, gate 1
    y, y_d = res[0], res[1]
    y_slack = res[2] if h_rel_err is not None else None
    n_amb = res[3] if h_rel_err is not None else 0
    for e in range(n_experts):
        rows = perm[offsets[e]:offsets[e + 1]]
        if rows.size == 0:
            continue
        res = expert_ffn(qx[rows], sx[rows], *get_expert(e), h_rel_err=h_rel_err)
        kpos = np.argmax(r["topk_idx"][rows] == e, axis=1)
        g = r["gates"][rows, kpos][:, None]
        y[rows] += g * res[0]
        y_d[rows] += g * res[1]
        if h_rel_err is not None:
            y_slack[rows] += g * res[2]
            n_amb += res[3]

    return {
        "qx": qx, "sx": sx, "logits64": z64, "logits_d": zd,
        "topk_idx": r["topk_idx"], "gates": r["gates"],
        "counts": counts, "offsets": offsets, "perm": perm, "inv": inv,
        "y": y, "y_d": y_d, "y_slack": y_slack, "n_ambiguous": n_amb,
    }
