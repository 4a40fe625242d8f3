"""Expert SwiGLU FFN on FP8 inputs and the DeepSeekMoE layer forward.

Test infrastructure: a plain float64 NumPy statement of what the layer
computes.  Only the tests, the smoke check and the benchmark's CPU baseline
use it; the HIP library never does.

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

The requantised a is decided from values that any implementation forms in
float32 (the recipe promotes the GEMM's partial sums to FP32), so a value
that sits within that rounding error of an E4M3 rounding point may come out
as another code.  requant_ambiguity gives, per element, the range of codes
that are valid under that error; a comparison then checks every code against
its range (a single code almost everywhere) and runs the down projection on
the codes the implementation actually produced (moe_layer's a_codes), so
that the layer output is held to the full bar with no allowance.
"""

import numpy as np

from .e4m3 import decode, encode
from .gemm import block_scaled_gemm, gemm_normaliser
from .quant import quant_act_1x128
from .route import permute, route

def expert_gate_up(qx, sx, q13, s13):
    """Gate/up projection, SwiGLU and the 1x128 requantisation of a.

    qx uint8 [n][H], sx f32 [n][H/128]; q13 uint8 [2I][H], s13 f32
    [2I/128][H/128].  Returns (h float64 [n][2I], a32 float32 [n][I],
    qa uint8 [n][I], sa float32 [n][I/128]).
    """
    inter = q13.shape[0] // 2
    h = block_scaled_gemm(qx, sx, q13, s13)                  # [n][2I]
    gate, up = h[:, :inter], h[:, inter:]
    with np.errstate(over="ignore"):
        a = gate / (1.0 + np.exp(-gate)) * up
    a32 = a.astype(np.float32)
    qa, sa = quant_act_1x128(a32)
    return h, a32, qa, sa


def requant_ambiguity(h, h_d, a32, qa, sa, h_rel_err):
    """Codes of a (and scales) that an implementation may legitimately set
    differently because it forms h in float32.

    h, h_d     float64 [n][2I]: the exact gate/up output and its normaliser
               |x_hat| . |w13_hat|^T
    a32, qa, sa  this oracle's a (float32) and its codes and scales
    h_rel_err  bound on |h_impl - h| / h_d

    An implementation's a differs from a32 by at most da (first-order
    propagation of the h error through silu(g) * u, plus a few float32 ulps
    of its own evaluation); its tile amax, hence its scale, moves by at most
    the tile's largest da.  The value v = a / s it encodes therefore lies
    within dv of this oracle's, and every code that rounds some value of
    [v - dv, v + dv] is a valid result (the encoder is monotone, so these
    are the codes from E4M3(v - dv) to E4M3(v + dv)).
    Returns (amb bool [n][I]: more than one valid code, lo and hi float64
    [n][I]: the values of the lowest and highest valid code, sa_tol float64
    [n][I/128]: the largest |s_impl - s|, the amax movement over 448 plus one
    float32 ulp of s for the rounding of the division).
    """
    inter = h.shape[1] // 2
    g, u = h[:, :inter], h[:, inter:]
    dg, du = h_rel_err * h_d[:, :inter], h_rel_err * h_d[:, inter:]
    with np.errstate(over="ignore"):
        sig = 1.0 / (1.0 + np.exp(-g))
    silu = g * sig
    dsilu = np.abs(sig * (1.0 + g * (1.0 - sig)))
    da = dsilu * dg * np.abs(u) + np.abs(silu) * du + dg * du + 8 * 2.0 ** -24 * np.abs(a32)
    n, cols = a32.shape
    tiles = cols // 128
    s = np.repeat(sa.astype(np.float64), 128, axis=1)
    amax_t = np.max(np.abs(a32.reshape(n, tiles, 128)), axis=2).astype(np.float64)
    da_t = np.max(da.reshape(n, tiles, 128), axis=2)
    amax = np.repeat(amax_t, 128, axis=1)
    da_tile = np.repeat(da_t, 128, axis=1)
    v = a32.astype(np.float64) / s
    # relative movement of the scale: delta = da_tile / amax; the other side's
    # v = a' / s' with |a' - a| <= da and s' >= s (1 - delta), so
    # |v' - v| <= (da / s + |v| delta) / (1 - delta); with delta >= 1 (a tile
    # whose amax is within the error) any code is possible
    with np.errstate(divide="ignore", invalid="ignore"):
        delta = np.where(da_tile == 0, 0.0, da_tile / amax)
        dv = np.where(delta < 1, (da / s + np.abs(v) * delta) / (1.0 - delta), np.inf)
    dv = dv + 2.0 ** -23 * np.abs(v)          # the float32 rounding of v -/+ dv below
    lo = decode(encode(np.maximum(v - dv, -448.0)))
    hi = decode(encode(np.minimum(v + dv, 448.0)))
    sa32 = np.asarray(sa, np.float32)
    sa_tol = da_t / 448.0 + np.spacing(sa32).astype(np.float64)
    return lo != hi, lo, hi, sa_tol


def expert_down(qa, sa, q2, s2):
    """Down projection o = a_hat . w2_hat^T and its normaliser |a_hat| . |w2_hat|^T.

    qa uint8 [n][I], sa f32 [n][I/128]; q2 uint8 [H][I], s2 f32
    [H/128][I/128].  Returns (o float64 [n][H], d float64 [n][H]).
    """
    return block_scaled_gemm(qa, sa, q2, s2), gemm_normaliser(qa, sa, q2, s2)


def expert_ffn(qx, sx, q13, s13, q2, s2):
    """One expert on quantised input rows: expert_gate_up then expert_down on
    its own codes.  Returns (o float64 [n][H], d float64 [n][H])."""
    _, _, qa, sa = expert_gate_up(qx, sx, q13, s13)
    return expert_down(qa, sa, q2, s2)


def router_logits(x, router_w):
    """z = x . Wr^T in float64, with its normaliser |x| . |Wr|^T."""
    x64 = np.asarray(x, np.float64)
    w64 = np.asarray(router_w, np.float64)
    return x64 @ w64.T, np.abs(x64) @ np.abs(w64).T


def moe_layer(x, router_w, bias, get_expert, shared, n_groups, groups_kept, top_k,
              logits=None, h_rel_err=None, a_codes=None):
    """DeepSeekMoE layer forward for the rows of x.

    x           float32 [T][H] holding bf16 values
    router_w    float32 [E][H] holding bf16 values
    bias        float32 [E]
    get_expert  callable e -> (q13, s13, q2, s2) for routed expert e
    shared      (q13, s13, q2, s2) of the shared expert
    logits      optional float32 [T][E]; when given, routing uses them instead
                of the oracle's own float64 logits rounded to float32
    h_rel_err   optional: also flag the codes of a that are decided within
                that relative error of h (requant_ambiguity)
    a_codes     optional dict with the down projection's FP8 input taken from
                elsewhere, token-major: "qa" uint8 [T][K][I], "sa" f32
                [T][K][I/128] (routed: token t's k-th expert) and "qa_sh",
                "sa_sh" ([T][I], [T][I/128]; the shared expert); when given,
                o and y are computed from these codes

    Returns a dict: qx, sx, logits64, logits_d, topk_idx, gates, counts,
    offsets, perm, inv, y (float64 [T][H]) and y_d (its normaliser), and this
    oracle's own codes of a in the same token-major layout (qa, sa, qa_sh,
    sa_sh; with h_rel_err also the requant_ambiguity results amb, lo, hi,
    sa_tol and amb_sh, lo_sh, hi_sh, sa_tol_sh, and n_ambiguous).
    """
    x = np.asarray(x, np.float32)
    t, h = x.shape
    n_experts = np.asarray(router_w).shape[0]
    qx, sx = quant_act_1x128(x)
    z64, zd = router_logits(x, router_w)
    z32 = z64.astype(np.float32) if logits is None else np.asarray(logits, np.float32)
    r = route(z32, bias, n_groups, groups_kept, top_k)
    counts, offsets, perm, inv = permute(r["topk_idx"], n_experts)

    inter = shared[0].shape[0] // 2
    own = {"qa": np.zeros((t, top_k, inter), np.uint8),
           "sa": np.zeros((t, top_k, inter // 128), np.float32)}
    if h_rel_err is not None:
        own["amb"] = np.zeros((t, top_k, inter), bool)
        own["lo"] = np.zeros((t, top_k, inter))
        own["hi"] = np.zeros((t, top_k, inter))
        own["sa_tol"] = np.zeros((t, top_k, inter // 128))

    def run(rows, weights):
        q13, s13, q2, s2 = weights
        hh, a32, qa, sa = expert_gate_up(qx[rows], sx[rows], q13, s13)
        flags = None
        if h_rel_err is not None:
            flags = requant_ambiguity(hh, gemm_normaliser(qx[rows], sx[rows], q13, s13),
                                      a32, qa, sa, h_rel_err)
        return qa, sa, flags

    # shared expert, gate 1
    all_rows = np.arange(t)
    qa, sa, flags = run(all_rows, shared)
    own.update({"qa_sh": qa, "sa_sh": sa})
    if h_rel_err is not None:
        own.update(dict(zip(("amb_sh", "lo_sh", "hi_sh", "sa_tol_sh"), flags)))
    src = a_codes if a_codes is not None else own
    y, y_d = expert_down(src["qa_sh"], src["sa_sh"], shared[2], shared[3])
    for e in range(n_experts):
        rows = perm[offsets[e]:offsets[e + 1]]
        if rows.size == 0:
            continue
        w = get_expert(e)
        kpos = np.argmax(r["topk_idx"][rows] == e, axis=1)
        qa, sa, flags = run(rows, w)
        own["qa"][rows, kpos] = qa
        own["sa"][rows, kpos] = sa
        if h_rel_err is not None:
            for k, f in zip(("amb", "lo", "hi", "sa_tol"), flags):
                own[k][rows, kpos] = f
        o, d = expert_down(src["qa"][rows, kpos], src["sa"][rows, kpos], w[2], w[3])
        g = r["gates"][rows, kpos][:, None]
        y[rows] += g * o
        y_d[rows] += g * d

    out = {
        "qx": qx, "sx": sx, "logits64": z64, "logits_d": zd,
        "topk_idx": r["topk_idx"], "gates": r["gates"],
        "counts": counts, "offsets": offsets, "perm": perm, "inv": inv,
        "y": y, "y_d": y_d,
    }
    out.update(own)
    if h_rel_err is not None:
        out["n_ambiguous"] = int(own["amb"].sum() + own["amb_sh"].sum())
    return out
