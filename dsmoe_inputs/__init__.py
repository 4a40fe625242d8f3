"""Seeded synthetic inputs shared by the tests, the smoke check and the
benchmark.

This module only draws numbers and lays them out; it holds none of the
layer's arithmetic (no quantisation, routing or GEMM).  The HIP library and
the CPU oracle both consume what it produces, byte for byte: small cases are
drawn with NumPy on the host, the DeepSeek-V3-sized weight sets (about 11 G
bf16 values) are drawn per expert with torch's seeded generator directly on
the device, and whatever the oracle needs of those is copied back to host.

Workloads (sizes of the DeepSeek-V3 MoE layer: hidden 7168, 256 routed
experts in 8 groups, 4 groups and 8 experts kept, one shared expert,
intermediate 2048):

  tiny        T=256,   H=512,  E=16,  G=4, Mg=2, K=2, I=256, bias 0
  dense       one GEMM M=4096, K=7168, N=4096, 1% of A entries x50 outliers
  v3_prefill  T=4096,  bias ~ U(-0.01, 0.01)
  v3_decode   T=64
  v3_skew     T=32768, router logits offset so expert popularity is Zipf(1.1)

x ~ N(0, 1), expert weights ~ N(0, 0.02), router weights ~ N(0, 0.006) for the
V3 shapes and N(0, 0.02) for the tiny case; all rounded to bf16 (nearest
even) before use.
"""

from __future__ import annotations

import dataclasses
import zlib

import numpy as np


@dataclasses.dataclass(frozen=True)
class LayerConfig:
    name: str
    T: int
    H: int
    E: int
    G: int
    Mg: int
    K: int
    I: int
    router_std: float
    weight_std: float = 0.02
    bias_range: float = 0.0        # bias ~ U(-r, r); 0 means b = 0
    zipf_s: float = 0.0            # > 0: skew expert popularity (see zipf_logit_offsets)
    zipf_beta: float = 0.5


LAYER_CONFIGS = {
    "tiny": LayerConfig("tiny", T=256, H=512, E=16, G=4, Mg=2, K=2, I=256, router_std=0.02),
    "v3_prefill": LayerConfig("v3_prefill", T=4096, H=7168, E=256, G=8, Mg=4, K=8, I=2048,
                              router_std=0.006, bias_range=0.01),
    "v3_decode": LayerConfig("v3_decode", T=64, H=7168, E=256, G=8, Mg=4, K=8, I=2048,
                             router_std=0.006, bias_range=0.01),
    "v3_skew": LayerConfig("v3_skew", T=32768, H=7168, E=256, G=8, Mg=4, K=8, I=2048,
                           router_std=0.006, bias_range=0.01, zipf_s=1.1),
}

DENSE_GEMM = dict(M=4096, K=7168, N=4096, outlier_frac=0.01, outlier_mult=50.0, b_std=0.02)


def _seed_words(name: str, seed: int):
    return [int(seed), zlib.crc32(name.encode("utf-8"))]


def rng(name: str, seed: int = 0) -> np.random.Generator:
    """Independent generator per (tensor name, seed)."""
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(_seed_words(name, seed))))


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 (ties to even); returns
    float32 holding bf16-representable values."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    bits = x.view(np.uint32).astype(np.uint64)
    bits = (bits + 0x7FFF + ((bits >> 16) & 1)) & 0xFFFF0000
    return bits.astype(np.uint32).view(np.float32).reshape(x.shape)


def normal_bf16(name: str, shape, std: float, seed: int = 0) -> np.ndarray:
    v = rng(name, seed).standard_normal(size=shape, dtype=np.float32) * np.float32(std)
    return bf16_round(v)


def uniform_f32(name: str, shape, lo: float, hi: float, seed: int = 0) -> np.ndarray:
    return rng(name, seed).uniform(lo, hi, size=shape).astype(np.float32)


def zipf_logit_offsets(n_experts: int, s: float, beta: float, seed: int = 0) -> np.ndarray:
    """Per-expert logit offset beta * ln p_r(e), with p_r proportional to
    r^-s over ranks r = 1..E and the rank of each expert a seeded permutation."""
    ranks = rng("zipf_rank", seed).permutation(n_experts) + 1
    p = ranks.astype(np.float64) ** (-s)
    p /= p.sum()
    return (beta * np.log(p)).astype(np.float32)


def layer_inputs_host(cfg: LayerConfig, seed: int = 0, with_weights: bool = True):
    """All inputs of one layer as host arrays (float32 holding bf16 values).

    Sized for small configs: the weights are E+1 expert sets of
    3*H*I values each.  Keys: x [T][H], router_w [E][H], bias [E],
    w13 [E+1][2I][H], w2 [E+1][H][I] (index E is the shared expert).
    """
    d = {
        "x": normal_bf16("x", (cfg.T, cfg.H), 1.0, seed),
        "router_w": normal_bf16("router_w", (cfg.E, cfg.H), cfg.router_std, seed),
        "bias": (uniform_f32("bias", (cfg.E,), -cfg.bias_range, cfg.bias_range, seed)
                 if cfg.bias_range > 0 else np.zeros(cfg.E, np.float32)),
    }
    if cfg.zipf_s > 0:
        apply_zipf_skew(d["x"], d["router_w"], cfg, seed)
    if with_weights:
        d["w13"] = normal_bf16("w13", (cfg.E + 1, 2 * cfg.I, cfg.H), cfg.weight_std, seed)
        d["w2"] = normal_bf16("w2", (cfg.E + 1, cfg.H, cfg.I), cfg.weight_std, seed)
    return d


def apply_zipf_skew(x: np.ndarray, router_w: np.ndarray, cfg: LayerConfig, seed: int = 0):
    """Bias the router logits through the inputs themselves: hidden channel 0
    of every token is set to 1 and router weight [e][0] to bf16(beta ln p_r(e)),
    so that x . Wr_e gains the Zipf offset of expert e (in place)."""
    off = zipf_logit_offsets(cfg.E, cfg.zipf_s, cfg.zipf_beta, seed)
    x[:, 0] = 1.0
    router_w[:, 0] = bf16_round(off)


def dense_gemm_inputs_host(m: int, n: int, k: int, seed: int = 0,
                           outlier_frac: float = 0.01, outlier_mult: float = 50.0,
                           b_std: float = 0.02):
    """A [M][K] ~ N(0,1) with a seeded outlier_frac of entries multiplied by
    outlier_mult, and B given transposed as W [N][K] ~ N(0, b_std); both bf16."""
    a = rng("dense_a", seed).standard_normal(size=(m, k), dtype=np.float32)
    n_out = int(round(outlier_frac * m * k))
    if n_out:
        idx = rng("dense_outliers", seed).choice(m * k, size=n_out, replace=False)
        a.reshape(-1)[idx] *= np.float32(outlier_mult)
    w = rng("dense_w", seed).standard_normal(size=(n, k), dtype=np.float32) * np.float32(b_std)
    return bf16_round(a), bf16_round(w)


# --------------------------------------------------------------------------
# Device-side generation for the DeepSeek-V3-sized weight sets (torch).
# --------------------------------------------------------------------------

def _torch_gen(name: str, seed: int, device):
    import torch
    g = torch.Generator(device=device)
    g.manual_seed((int(seed) << 32) ^ zlib.crc32(name.encode("utf-8")))
    return g


def expert_weights_device(cfg: LayerConfig, e: int, device, seed: int = 0):
    """bf16 (w13 [2I][H], w2 [H][I]) of routed expert e (e == E: the shared
    expert), drawn on the device from a generator seeded per expert."""
    import torch
    g = _torch_gen(f"expert{e}", seed, device)
    w13 = torch.randn((2 * cfg.I, cfg.H), generator=g, device=device, dtype=torch.float32)
    w13.mul_(cfg.weight_std)
    w2 = torch.randn((cfg.H, cfg.I), generator=g, device=device, dtype=torch.float32)
    w2.mul_(cfg.weight_std)
    return w13.to(torch.bfloat16), w2.to(torch.bfloat16)


def layer_activations_device(cfg: LayerConfig, device, seed: int = 0):
    """x [T][H] bf16, router_w [E][H] bf16, bias [E] f32 on the device.
    Drawn on the host with NumPy (small next to the weights) and copied."""
    import torch
    d = layer_inputs_host(cfg, seed, with_weights=False)
    return (torch.from_numpy(d["x"]).to(torch.bfloat16).to(device),
            torch.from_numpy(d["router_w"]).to(torch.bfloat16).to(device),
            torch.from_numpy(d["bias"]).to(device))
