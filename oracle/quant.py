"""Fine-grained online FP8 quantisation: 1x128 activation tiles, 128x128
weight blocks.

Source: V3 notes §6.1 (activations scaled per 1x128 tile -- one scale per
token per 128 channels; weights per 128x128 block; scales computed online from
the tensor itself rather than predicted from history); the same two
granularities in the infra answer (FP8 paragraph, "per-tile (1x128) and
per-group (128x128)") and in the evolution post (V3 FP8 section).

Readings taken where the pages are silent (each is also listed with the
design notes of the repository):

* scale  s = fl32(amax / 448) by IEEE float32 division, amax = max |x| over
  the tile taken exactly in float32; the scale is not rounded to a power of 2;
* an all-zero tile (amax == 0) gets s = 1.0;
* codes  q = E4M3(fl32(x / s)) with IEEE float32 division (not a reciprocal
  multiply), round half to even, saturating;
* no flush of float32 subnormals anywhere.
"""

import numpy as np

from .e4m3 import encode

TILE = 128
FP8_MAX = np.float32(448.0)


def _scale_from_amax(amax: np.ndarray) -> np.ndarray:
    amax = np.asarray(amax, dtype=np.float32)
    s = (amax / FP8_MAX).astype(np.float32)          # IEEE float32 division
    return np.where(amax == 0, np.float32(1.0), s).astype(np.float32)


def quant_act_1x128(x: np.ndarray):
    """Quantise x[rows][cols] per 1x128 tile.

    Returns (q uint8 [rows][cols], s float32 [rows][cols/128]).
    Input values must be exactly representable in float32 (bf16 or f32 data).
    """
    x = np.asarray(x, dtype=np.float32)
    rows, cols = x.shape
    if cols % TILE:
        raise ValueError("cols must be a multiple of 128")
    tiles = x.reshape(rows, cols // TILE, TILE)
    amax = np.max(np.abs(tiles), axis=2) if rows and cols else np.zeros((rows, cols // TILE), np.float32)
    s = _scale_from_amax(amax)
    scaled = (tiles / s[:, :, None]).astype(np.float32)   # IEEE float32 division
    q = encode(scaled).reshape(rows, cols)
    return q, s


def quant_w_128x128(w: np.ndarray):
    """Quantise w[n_mats][N][K] (or [N][K]) per 128x128 block.

    Returns (q uint8 same shape, s float32 [n_mats][N/128][K/128]).
    """
    w = np.asarray(w, dtype=np.float32)
    squeeze = w.ndim == 2
    if squeeze:
        w = w[None]
    nm, n, k = w.shape
    if n % TILE or k % TILE:
        raise ValueError("N and K must be multiples of 128")
    blocks = w.reshape(nm, n // TILE, TILE, k // TILE, TILE)
    amax = np.max(np.abs(blocks), axis=(2, 4)) if w.size else np.zeros((nm, n // TILE, k // TILE), np.float32)
    s = _scale_from_amax(amax)                             # [nm][N/128][K/128]
    scaled = (blocks / s[:, :, None, :, None]).astype(np.float32)
    q = encode(scaled).reshape(nm, n, k)
    if squeeze:
        return q[0], s[0]
    return q, s
