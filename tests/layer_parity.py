"""The layer parity protocol shared by the GPU layer tests and the smoke check
(not collected: no test_ prefix).

Every checked token is held to:
* qx / sx (the 1x128 codes of x): bit-exact;
* logits: |gpu - oracle| <= LOGIT_TOL * (|x| . |Wr|^T).  The GPU sums bf16
  products (exact in FP32) in FP32 over H/32 MFMA steps; the bound is the
  FP32 summation error of that depth, (H/32 + 5) * 2^-24 = 1.4e-5 at
  H = 7168, rounded up;
* routing: the oracle routes on the GPU's logits (the check above bounds how
  far they are from its own), so topk_idx, counts, offsets, perm and inv
  must match bit for bit; gates within 1e-6;
* a, the requantised SwiGLU output (the down projection's FP8 input): every
  code equals the oracle's, except where the FP32 error of h (H_REL_ERR)
  allows more than one code (requant_ambiguity); there the code must lie in
  the allowed range; scales lie within the bound;
* y: the oracle's down projections and combine run on the GPU's own codes
  of a, and max |gpu - oracle| / y_d <= 2e-3 (float32 y) or 1e-2 (bf16 y),
  y_d = sum_k gate_k |a_hat| . |w2_hat|^T plus the shared expert's term.
"""

import numpy as np

from oracle import e4m3 as oe
from oracle import gemm as og
from oracle import layer as ol
from oracle import quant as oq
from oracle import route as orr

LOGIT_TOL = 2e-5
# Bound on the GPU's error in h = x W13^T relative to |x_hat| . |w13_hat|:
# per 128-wide chunk, the sum of its exact FP8 products in FP32 (at most
# 127 roundings, each <= 2^-24 of the chunk's sum of |products|), the
# rounding of the scale product sa * sw and of the promoting FMA; over the
# H/128 = 56 chunks the accumulator's own roundings add at most 56 * 2^-24 of
# the running |total| <= |x_hat| . |w13_hat|.  (127 + 1 + 56) * 2^-24 =
# 1.10e-5, rounded up.
H_REL_ERR = 1.2e-5
Y_TOL = {"f32": 2e-3, "bf16": 1e-2}


def normalised_error(got, want, norm, what):
    """max |got - want| / norm (where norm == 0 the values must be equal)."""
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    norm = np.asarray(norm, np.float64)
    err = np.abs(got - want)
    zero = norm == 0
    assert np.all(err[zero] == 0), f"{what}: non-zero error where the normaliser is 0"
    rel = np.where(zero, 0.0, err / np.where(zero, 1.0, norm))
    return float(rel.max()) if rel.size else 0.0


def assert_close(got, want, norm, tol, what):
    worst = normalised_error(got, want, norm, what)
    print(f"[parity] {what}: max normalised error {worst:.3e} (tolerance {tol:.1e})", flush=True)
    assert worst <= tol, f"{what}: max normalised error {worst:.3e} > {tol:.1e}"
    return worst


def check_codes(got_q, got_s, want, what, sfx=""):
    """Codes of a against the oracle's: every GPU code lies in the range of
    valid codes requant_ambiguity gives (the oracle's own code wherever the
    range is a single code); scales within the bound.  want holds qa, lo, hi,
    amb, sa, sa_tol (with suffix sfx).  Returns (flagged, differing)."""
    got_q = np.asarray(got_q)
    want_q = want["qa" + sfx]
    lo, hi, amb = want["lo" + sfx], want["hi" + sfx], want["amb" + sfx]
    gv = oe.decode(got_q)
    bad = (gv < lo) | (gv > hi)
    assert not bad.any(), \
        f"{what}: {int(bad.sum())} codes of a lie outside the range the FP32 error of h allows, e.g. " + \
        ", ".join(f"gpu {int(a):#04x} vs oracle {int(b):#04x} (valid {l:.4g}..{h:.4g})" for a, b, l, h in
                  zip(got_q[bad][:6], want_q[bad][:6], lo[bad][:6], hi[bad][:6]))
    differ = got_q != want_q
    # a code that differs must be flagged (+0 and -0 decode alike)
    assert not np.any(differ & ~amb & (gv != oe.decode(want_q))), f"{what}: an unflagged code differs"
    serr = np.abs(np.asarray(got_s, np.float64) - np.asarray(want["sa" + sfx], np.float64))
    tol = want["sa_tol" + sfx]
    assert np.all(serr <= tol), f"{what}: a scale of a is off by more than its bound " \
                                f"(worst excess {float((serr - tol).max()):.3e})"
    n_amb, n_diff = int(amb.sum()), int(differ.sum())
    print(f"[parity] {what}: {differ.size} codes of a, {n_amb} with more than one valid code, {n_diff} "
          f"differ from the oracle's (all within their valid range); scales within bound", flush=True)
    return n_amb, n_diff


def gpu_a_codes(g, T, K, toks, n_shared, inter):
    """The GPU's codes of a for tokens `toks`, token-major as moe_layer's
    a_codes: row inv[t][k] for routed pair (t, k), row T*K + t for the shared
    expert."""
    inv = g["inv"][toks]
    out = {"qa": g["qa"][inv], "sa": g["sa"][inv]}
    if n_shared:
        out["qa_sh"] = g["qa"][T * K + toks]
        out["sa_sh"] = g["sa"][T * K + toks]
    else:      # the oracle's zero stand-in for a missing shared expert: codes 0, scale 1
        out["qa_sh"] = np.zeros((len(toks), inter), np.uint8)
        out["sa_sh"] = np.ones((len(toks), inter // 128), np.float32)
    return out


def check_routing_all(g, bias, G, Mg, K, E, what):
    """Oracle routing and permute of every token on the GPU's logits against
    the GPU's: bit-exact indices, counts, offsets, perm, inv; gates 1e-6."""
    r = orr.route(g["logits"], bias, G, Mg, K)
    counts, offsets, perm, inv = orr.permute(r["topk_idx"], E)
    assert np.array_equal(g["topk_idx"], r["topk_idx"]), f"{what}: topk_idx differs"
    assert np.array_equal(g["counts"], counts), f"{what}: counts differ"
    assert np.array_equal(g["offsets"], offsets), f"{what}: offsets differ"
    assert np.array_equal(g["perm"], perm), f"{what}: perm differs"
    assert np.array_equal(g["inv"], inv), f"{what}: inv differs"
    gerr = float(np.abs(g["gates"] - r["gates"]).max(initial=0.0))
    assert gerr <= 1e-6, f"{what}: gates differ by {gerr:.2e}"
    print(f"[parity] {what}: routing of {len(g['topk_idx'])} tokens bit-exact "
          f"(indices, counts, offsets, perm, inv; gates within {gerr:.1e})", flush=True)
    return r, (counts, offsets, perm, inv)


def check_tokens(g, y_gpu, want, toks, T, K, n_shared, out_dtype, what):
    """Per-token checks of a layer forward against moe_layer's result for the
    tokens `toks` (routed on the GPU's logits, down projection on the GPU's
    codes of a)."""
    assert np.array_equal(g["qx"][toks], want["qx"]), f"{what}: qx differs"
    assert np.array_equal(g["sx"][toks].view(np.uint32), want["sx"].view(np.uint32)), f"{what}: sx differs"
    assert_close(g["logits"][toks], want["logits64"], want["logits_d"], LOGIT_TOL, f"{what} logits")
    assert np.array_equal(g["topk_idx"][toks], want["topk_idx"]), f"{what}: topk_idx differs"
    assert float(np.abs(g["gates"][toks] - want["gates"]).max(initial=0.0)) <= 1e-6
    codes = gpu_a_codes(g, T, K, toks, n_shared, want["qa"].shape[2])
    check_codes(codes["qa"], codes["sa"], want, f"{what} routed a")
    if n_shared:
        check_codes(codes["qa_sh"], codes["sa_sh"], want, f"{what} shared a", "_sh")
    return assert_close(y_gpu[toks], want["y"], want["y_d"], Y_TOL[out_dtype], f"{what} y")


def check_group_codes(g, x, rows, toks, q13, s13, what):
    """Codes of a over whole GEMM row ranges: GPU rows `rows` of qa/sa hold
    tokens `toks` of one expert (q13, s13); the oracle forms them from x."""
    qx, sx = oq.quant_act_1x128(x[toks])
    h, a32, qa, sa = ol.expert_gate_up(qx, sx, q13, s13)
    amb, lo, hi, tol = ol.requant_ambiguity(h, og.gemm_normaliser(qx, sx, q13, s13), a32, qa, sa, H_REL_ERR)
    want = {"qa": qa, "sa": sa, "amb": amb, "lo": lo, "hi": hi, "sa_tol": tol}
    return check_codes(g["qa"][rows], g["sa"][rows], want, what)
