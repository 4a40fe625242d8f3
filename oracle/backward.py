"""Pieces of the FP8 backward of the expert FFN: the data-gradient (dgrad)
GEMMs on block-transposed weights.

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

from .gemm import grouped_gemm


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
