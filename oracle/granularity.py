"""Scaling-granularity study: FP8 E4M3 GEMM error of three scale layouts.

Test infrastructure: imported only by the tests, the smoke check and the
benchmark's CPU baseline; the library never uses it.

Source: infra answer (51itzy.com), FP8 paragraph.  Coarse per-tensor E4M3
scaling lets single outliers inflate the quantisation error of a whole
tensor, fine-grained 1x128 / 128x128 scaling is the recipe's answer, and
per-token x per-channel scaling, simpler to implement, is named as not
discussed.  V3 notes §6.1 give the fine-grained recipe itself.

Granularities (activation A [M][K], weight W [N][K], both contracted over K):

* ``tensor``:  one scale for all of A, one for all of W;
* ``channel``: one scale per row of A (per token) and one per row of W
  (per output channel), each over the whole contraction axis;
* ``block``:   1x128 tiles of A and 128x128 blocks of W (the recipe).

Every scale follows the same rule as the recipe's quantisers: s = fl32(amax /
448) by IEEE float32 division (s = 1 when amax = 0), codes E4M3(fl32(x / s))
by IEEE division, round half to even, saturating.  The GEMM of the
dequantised operands is evaluated in float64; the reference is the float64
product of the unquantised (bf16) inputs.
"""

import numpy as np

from .e4m3 import decode, encode
from .gemm import dequant_act, dequant_w
from .quant import TILE, quant_act_1x128, quant_w_128x128

FP8_MAX = np.float32(448.0)
GRANULARITIES = ("tensor", "channel", "block")


def _scale(amax) -> np.ndarray:
    amax = np.asarray(amax, dtype=np.float32)
    s = (amax / FP8_MAX).astype(np.float32)
    return np.where(amax == 0, np.float32(1.0), s).astype(np.float32)


def quant_tensor(x: np.ndarray):
    """One scale for the whole tensor.  Returns (q uint8, s float32 scalar)."""
    x = np.asarray(x, dtype=np.float32)
    amax = np.max(np.abs(x)) if x.size else np.float32(0.0)
    s = _scale(amax)
    return encode((x / s).astype(np.float32)), np.float32(s)


def quant_rows(x: np.ndarray):
    """One scale per row over the whole row (per token for an activation,
    per output channel for a weight stored [N][K]).
    Returns (q uint8 [rows][cols], s float32 [rows])."""
    x = np.asarray(x, dtype=np.float32)
    amax = np.max(np.abs(x), axis=1) if x.size else np.zeros((x.shape[0],), np.float32)
    s = _scale(amax)
    return encode((x / s[:, None]).astype(np.float32)), s


def dequantised(a: np.ndarray, w: np.ndarray, granularity: str):
    """(A_hat, W_hat) in float64 after quantising a [M][K] and w [N][K] at
    the given granularity."""
    if granularity == "tensor":
        qa, sa = quant_tensor(a)
        qw, sw = quant_tensor(w)
        return decode(qa) * np.float64(sa), decode(qw) * np.float64(sw)
    if granularity == "channel":
        qa, sa = quant_rows(a)
        qw, sw = quant_rows(w)
        return decode(qa) * sa.astype(np.float64)[:, None], decode(qw) * sw.astype(np.float64)[:, None]
    if granularity == "block":
        qa, sa = quant_act_1x128(a)
        qw, sw = quant_w_128x128(w)
        return dequant_act(qa, sa), dequant_w(qw, sw)
    raise ValueError(f"unknown granularity {granularity!r}")


def gemm_errors(a: np.ndarray, w: np.ndarray, granularity: str) -> dict:
    """Error of C_hat = A_hat W_hat^T against C = A W^T (float64 of the given
    inputs): max and mean of |C_hat - C| / (|A| |W|^T) element-wise, and the
    relative Frobenius error ||C_hat - C|| / ||C||."""
    a64 = np.asarray(a, dtype=np.float64)
    w64 = np.asarray(w, dtype=np.float64)
    ah, wh = dequantised(a, w, granularity)
    c = a64 @ w64.T
    ch = ah @ wh.T
    d = np.abs(a64) @ np.abs(w64).T
    err = np.abs(ch - c)
    rel = np.where(d > 0, err / np.where(d > 0, d, 1.0), 0.0)
    return {
        "max_norm_err": float(rel.max()),
        "mean_norm_err": float(rel.mean()),
        "rel_frobenius": float(np.linalg.norm(ch - c) / np.linalg.norm(c)),
    }


def operand_errors(x: np.ndarray, granularity: str, weight: bool = False) -> dict:
    """Quantisation error of one operand: relative Frobenius error of the
    dequantised tensor and the fraction of non-zero values quantised to 0."""
    x = np.asarray(x, dtype=np.float32)
    if granularity == "tensor":
        q, s = quant_tensor(x)
        xh = decode(q) * np.float64(s)
    elif granularity == "channel":
        q, s = quant_rows(x)
        xh = decode(q) * s.astype(np.float64)[:, None]
    elif granularity == "block":
        if weight:
            q, s = quant_w_128x128(x)
            xh = dequant_w(q, s)
        else:
            q, s = quant_act_1x128(x)
            xh = dequant_act(q, s)
    else:
        raise ValueError(f"unknown granularity {granularity!r}")
    x64 = x.astype(np.float64)
    nz = x64 != 0
    return {
        "rel_frobenius": float(np.linalg.norm(xh - x64) / np.linalg.norm(x64)),
        "flushed_to_zero": float(np.mean((xh == 0) & nz) / max(np.mean(nz), 1e-300)),
    }


__all__ = ["GRANULARITIES", "quant_tensor", "quant_rows", "dequantised", "gemm_errors",
           "operand_errors", "TILE"]
