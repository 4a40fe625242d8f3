"""The FP8 backward of the expert FFN: the data-gradient (dgrad) GEMMs on
block-transposed weights, the weight-gradient (Wgrad) GEMMs over each
expert's tokens, the SwiGLU backward on the recomputed activation, and the
gradients of the gates and the router logits.

Test infrastructure: imported only by the tests, the smoke check and the
benchmark's CPU baseline; the library never uses it.

Sources: V3 notes §6 (the forward, the activation-gradient and the
weight-gradient GEMMs all run in FP8, E4M3 throughout) and §6.1 (1x128 tiles
for activations, 128x128 blocks for weights).  The pages do not orient the
gradient tiles; the plainest reading, taken here, is 1x128 along each GEMM's
contraction axis for the gradient operand, and the forward's 128x128 weight
blocks for the weights.

For the down projection z = a W2^T (W2 [H][I]) the data gradient is
da = dz W2: contraction over H, so dz is quantised in 1x128 tiles along H and
the weight operand, stored [N][K] like every weight, is W2^T [I][H].  For the
gate/up projection h = x W13^T (W13 [2I][H]), dx = dh W13 with W13^T [H][2I].
A 128x128 block's amax does not change under transposition, so the weight
operand of a dgrad GEMM is the transposed codes and the transposed block
scales of the forward's weight, with no new quantisation (the pins check
that against quantising W^T directly).
"""

import numpy as np

from .e4m3 import decode
from .gemm import grouped_gemm
from .quant import quant_act_1x128
from .route import affinity


def transpose_blocks(q: np.ndarray, s: np.ndarray):
    """Codes [n][N][K] and 128x128 scales [n][N/128][K/128] of W -> those of
    W^T: codes [n][K][N], scales [n][K/128][N/128]."""
    return np.ascontiguousarray(np.swapaxes(q, -1, -2)), np.ascontiguousarray(np.swapaxes(s, -1, -2))


def dgrad_grouped(qg, sg, g_rows, offsets, qw, sw):
    """Data gradient of a grouped GEMM c = A W_g^T: dA[r] = dC[r] . W_g, from
    the 1x128 codes qg / scales sg of dC (rows gathered by g_rows, as in the
    forward) and the forward's weight codes qw [G][N][K] / scales sw.  Returns
    float64 [rows][K]."""
    qt, st = transpose_blocks(qw, sw)
    return grouped_gemm(qg, sg, g_rows, offsets, qt, st)


__all__ = ["transpose_blocks", "dgrad_grouped"]


# ---------------------------------------------------------------------------
# Weight gradients, the SwiGLU backward and the gate / router gradients
# ---------------------------------------------------------------------------
#
# Weight-gradient (Wgrad) GEMMs contract over the tokens of each expert:
# dW2_e = sum over the expert's rows r of do[r] (x) a[r]  ([H][I]) and
# dW13_e = sum_r dh[r] (x) x[t_r]  ([2I][H]).  Read the same way as the dgrad
# tiles, both operands are quantised in 1x128 tiles along the contraction
# axis, i.e. 128 consecutive rows of one expert's group per tile (per column),
# starting at the group's first row; a group's last tile may be shorter.
#
# The SwiGLU output is recomputed in the backward from its input h (the infra
# answer's memory paragraph lists SwiGLU among the selectively recomputed
# operations), and its derivative is taken on that recomputation.
#
# The gates multiply the experts' outputs in higher precision, not in a GEMM:
# dgate[t,k] = <dy[t], o_k[t]> with o_k the ungated output of token t's k-th
# expert.  gate_k = s_k / sum_j s_j over the chosen experts and s = sigmoid(z)
# (the readings of the forward), so the router logits receive
# dz_e = s_e (1 - s_e) (dgate_e - sum_j dgate_j gate_j) / sum_j s_j for the
# chosen experts and nothing for the others; the bias b, used only to select,
# receives no gradient (it is moved by the balancing rule instead).


def chunk_offsets(offsets) -> np.ndarray:
    """Start of each group's first 128-row tile: exclusive scan of
    ceil(n_g / 128) (G+1 entries)."""
    offsets = np.asarray(offsets, np.int64)
    n = np.diff(offsets)
    return np.concatenate([[0], np.cumsum((n + 127) // 128)])


def quant_tokens_128(v, offsets):
    """1x128 tiles along the token axis inside each group.

    v float32 [rows][C] with the rows in group order (group g: rows
    offsets[g] .. offsets[g+1]-1), C a multiple of 128.  Tile j of group g
    covers its rows 128j .. 128j+127 (fewer in the last tile) of one column.
    Returns (q uint8 [rows][C], s float32 [n_tiles][C]) where row
    chunk_offsets(offsets)[g] + j of s holds the scales of tile j of group g.
    A short tile is quantised as if padded with zeros, which changes no amax.
    """
    v = np.asarray(v, np.float32)
    offsets = np.asarray(offsets, np.int64)
    rows, cols = v.shape
    cho = chunk_offsets(offsets)
    q = np.zeros((rows, cols), np.uint8)
    s = np.ones((int(cho[-1]), cols), np.float32)
    for g in range(len(offsets) - 1):
        for j, r0 in enumerate(range(int(offsets[g]), int(offsets[g + 1]), 128)):
            r1 = min(r0 + 128, int(offsets[g + 1]))
            tile = np.zeros((128, cols), np.float32)
            tile[:r1 - r0] = v[r0:r1]
            qt, st = quant_act_1x128(np.ascontiguousarray(tile.T))     # [cols][128], [cols][1]
            q[r0:r1] = qt.T[:r1 - r0]
            s[cho[g] + j] = st[:, 0]
    return q, s


def dequant_tokens_128(q, s, offsets) -> np.ndarray:
    """float64 values of quant_tokens_128 codes: q[r][c] * s[tile(r)][c]."""
    offsets = np.asarray(offsets, np.int64)
    cho = chunk_offsets(offsets)
    out = decode(q)
    for g in range(len(offsets) - 1):
        for j, r0 in enumerate(range(int(offsets[g]), int(offsets[g + 1]), 128)):
            r1 = min(r0 + 128, int(offsets[g + 1]))
            out[r0:r1] *= np.asarray(s[cho[g] + j], np.float64)[None, :]
    return out


def wgrad_grouped(qg, sg, qa, sa, offsets):
    """Weight gradient of a grouped GEMM c = A W_g^T over each group's rows:
    dW_g[n][k] = sum over rows r of group g of dC_hat[r][n] * A_hat[r][k],
    from codes with 1x128 tiles along the rows (quant_tokens_128): dC codes
    qg [rows][N] / scales sg, A codes qa [rows][K] / scales sa.
    Returns (dW float64 [G][N][K], its normaliser |dC_hat|^T |A_hat|)."""
    offsets = np.asarray(offsets, np.int64)
    dc = dequant_tokens_128(qg, sg, offsets)
    a = dequant_tokens_128(qa, sa, offsets)
    groups = len(offsets) - 1
    dw = np.zeros((groups, dc.shape[1], a.shape[1]))
    dn = np.zeros_like(dw)
    for g in range(groups):
        r0, r1 = int(offsets[g]), int(offsets[g + 1])
        dw[g] = dc[r0:r1].T @ a[r0:r1]
        dn[g] = np.abs(dc[r0:r1]).T @ np.abs(a[r0:r1])
    return dw, dn


def swiglu_backward(h, da):
    """Gradient of a = silu(h_gate) * h_up (h [n][2I]: gate columns, then up)
    given da [n][I], in float64: dh_gate = da * h_up * silu'(h_gate),
    dh_up = da * silu(h_gate), silu'(v) = sig(v) (1 + v (1 - sig(v)))."""
    h = np.asarray(h, np.float64)
    da = np.asarray(da, np.float64)
    inter = h.shape[1] // 2
    g, u = h[:, :inter], h[:, inter:]
    with np.errstate(over="ignore"):
        sig = 1.0 / (1.0 + np.exp(-g))
    return np.concatenate([da * u * sig * (1.0 + g * (1.0 - sig)), da * g * sig], axis=1)


def gate_backward(dy, o, topk_idx, logits, n_experts):
    """Gradients of y[t] = sum_k gate_k(t) o_k[t] (+ the shared expert) with
    respect to the gates and the router logits, routing held fixed.

    dy [T][H]; o [T][K][H] the ungated outputs of token t's chosen experts;
    topk_idx [T][K]; logits float32 [T][E] (the routing's own).  Returns
    (dgate float64 [T][K], dlogits float64 [T][E]) with
    dgate[t,k] = <dy[t], o[t,k]> and dlogits as in the notes above.
    """
    dy = np.asarray(dy, np.float64)
    o = np.asarray(o, np.float64)
    s = affinity(logits).astype(np.float64)
    s_sel = np.take_along_axis(s, np.asarray(topk_idx, np.int64), axis=1)
    tot = s_sel.sum(axis=1, keepdims=True)
    gates = s_sel / tot
    dgate = np.einsum("th,tkh->tk", dy, o)
    ds = (dgate - np.sum(dgate * gates, axis=1, keepdims=True)) / tot
    dz = np.zeros((dy.shape[0], n_experts))
    np.put_along_axis(dz, np.asarray(topk_idx, np.int64), ds * s_sel * (1.0 - s_sel), axis=1)
    return dgate, dz


__all__ += ["chunk_offsets", "quant_tokens_128", "dequant_tokens_128", "wgrad_grouped",
            "swiglu_backward", "gate_backward"]
