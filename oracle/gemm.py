"""Block-scaled FP8 GEMM with per-128-K promotion, in float64.

Source: V3 notes §6.2 -- after every 128 FP8 products the partial sum is
promoted and accumulated in FP32 (the report's remedy for the limited FP8
accumulation precision of Hopper tensor cores); the evolution post (V3 FP8
section) states the same low-precision-multiply / high-precision-accumulate
split.  With 1x128 activation scales and 128x128 weight scales (V3 notes
§6.1) every 128-wide K chunk carries its own pair of scales, so the promoted
partial sum of chunk c is multiplied by  sa[m, c] * sw[n // 128, c]  before it
is added to the running total.

Here each chunk's partial sum of decoded FP8 products is formed in float64,
where it is exact (every product of two E4M3 values is a multiple of 2^-18
below 2^18, so a sum of 128 of them needs at most 43 bits), then scaled and
accumulated in float64.  The result is the exact real value of the
block-scaled computation up to float64 rounding of the scaled accumulation.
"""

import numpy as np

from .e4m3 import decode

TILE = 128


def dequant_act(q: np.ndarray, s: np.ndarray) -> np.ndarray:
    """float64 values of 1x128-tiled codes: q[rows][cols] * s[rows][cols/128]."""
    return decode(q) * np.repeat(np.asarray(s, np.float64), TILE, axis=1)


def dequant_w(q: np.ndarray, s: np.ndarray) -> np.ndarray:
    """float64 values of 128x128-blocked codes: q[N][K] * s[N/128][K/128]."""
    s64 = np.asarray(s, np.float64)
    return decode(q) * np.repeat(np.repeat(s64, TILE, axis=0), TILE, axis=1)


def block_scaled_gemm(qa, sa, qw, sw) -> np.ndarray:
    """C[m][n] = sum over chunks c of sa[m,c] * sw[n//128,c] * P_c[m,n],
    P_c[m,n] = sum_{k in chunk c} dec(qa[m,k]) * dec(qw[n,k]).

    qa uint8 [M][K], sa f32 [M][K/128], qw uint8 [N][K] (output channel x
    input channel), sw f32 [N/128][K/128].  Returns float64 [M][N].
    """
    qa = np.asarray(qa)
    qw = np.asarray(qw)
    m, k = qa.shape
    n = qw.shape[0]
    a = decode(qa)
    w = decode(qw)
    sa64 = np.asarray(sa, np.float64)
    sw64 = np.asarray(sw, np.float64)
    c_out = np.zeros((m, n), dtype=np.float64)
    for c in range(k // TILE):
        ks = slice(c * TILE, (c + 1) * TILE)
        partial = a[:, ks] @ w[:, ks].T                         # exact
        scale = sa64[:, c][:, None] * np.repeat(sw64[:, c], TILE)[None, :]
        c_out += scale * partial
    return c_out


def gemm_normaliser(qa, sa, qw, sw) -> np.ndarray:
    """D[m][n] = sum_k |a_hat[m,k]| * |w_hat[n,k]| (the error normaliser)."""
    return np.abs(dequant_act(qa, sa)) @ np.abs(dequant_w(qw, sw)).T


def grouped_gemm(qa, sa, a_rows, offsets, qw, sw):
    """Grouped GEMM: for group g, output rows offsets[g]..offsets[g+1]-1 are
    A[a_rows[r]] x W_g^T (a_rows None means row r of A itself).

    qw uint8 [G][N][K], sw f32 [G][N/128][K/128].
    Returns (C float64 [M_total][N], D float64 [M_total][N]).
    """
    offsets = np.asarray(offsets, dtype=np.int64)
    groups = len(offsets) - 1
    m_total = int(offsets[-1])
    n = qw.shape[1]
    c_out = np.zeros((m_total, n), dtype=np.float64)
    d_out = np.zeros((m_total, n), dtype=np.float64)
    for g in range(groups):
        r0, r1 = int(offsets[g]), int(offsets[g + 1])
        if r1 <= r0:
            continue
        rows = np.arange(r0, r1) if a_rows is None else np.asarray(a_rows[r0:r1], dtype=np.int64)
        c_out[r0:r1] = block_scaled_gemm(qa[rows], sa[rows], qw[g], sw[g])
        d_out[r0:r1] = gemm_normaliser(qa[rows], sa[rows], qw[g], sw[g])
    return c_out, d_out
