"""GPU parity of the decode-serving bookkeeping (dsmoe_plan_replicas,
dsmoe_slot_offsets, dsmoe_place_replicas) against oracle.serving: plans,
offsets and placed weights must match bit for bit.  The serving forward's
output is checked against the oracle's layer in test_gpu_layer.py."""

import numpy as np
import pytest
import torch

from gpu_util import banner, dev, host
from oracle import serving as osv

pytestmark = pytest.mark.gpu


def _d():
    import fp8_block_scaled_dsmoe_amd as d
    return d


def _loads(kind, E, seed):
    r = np.random.default_rng(seed)
    if kind == "zipf":   # the skewed workload's popularity, 64 tokens x 8
        p = 1.0 / np.arange(1, E + 1) ** 1.1
        p = p[r.permutation(E)]
        return np.bincount(r.choice(E, size=512, p=p / p.sum()), minlength=E).astype(np.int32)
    if kind == "uniform":
        return r.integers(0, 40, E).astype(np.int32)
    if kind == "ties":
        return np.full(E, 7, np.int32)
    if kind == "zeros":
        return np.zeros(E, np.int32)
    return (r.integers(0, 2, E) * r.integers(1, 100000, E)).astype(np.int32)   # sparse, large


@pytest.mark.parametrize("kind", ["zipf", "uniform", "ties", "zeros", "sparse"])
@pytest.mark.parametrize("E,R", [(1, 0), (1, 5), (16, 6), (256, 0), (256, 64), (1000, 1024), (1024, 31)])
def test_plan_matches_oracle(kind, E, R):
    banner(f"plan_replicas {kind} E={E} R={R}")
    c = _loads(kind, E, seed=E + R)
    sf, se = _d().plan_replicas(dev(c), R)
    _, sf_o, se_o = osv.plan_replicas(c, R)
    assert np.array_equal(host(sf), sf_o)
    assert np.array_equal(host(se), se_o)


@pytest.mark.parametrize("E,R,extra", [(4, 3, -1), (16, 6, 256), (256, 64, 64), (256, 64, -1)])
def test_slot_offsets_match_oracle(E, R, extra):
    banner(f"slot_offsets E={E} R={R} extra={extra}")
    c = _loads("zipf", E, seed=R)
    off = np.concatenate([[0], np.cumsum(c)]).astype(np.int32)
    sf, se = _d().plan_replicas(dev(c), R)
    phys = host(_d().slot_offsets(dev(off), sf, se, extra))
    want = osv.physical_offsets(off, osv.plan_replicas(c, R)[1])
    S = E + R
    assert np.array_equal(phys[:S + 1], want)
    if extra >= 0:
        assert phys[S + 1] == off[-1] + extra


def test_place_replicas_copies_each_slot():
    banner("place_replicas")
    E, N, K = 6, 256, 384
    r = np.random.default_rng(5)
    w = r.integers(0, 256, (E, N, K), dtype=np.uint8)
    s = r.random((E, N // 128, K // 128)).astype(np.float32)
    c = np.array([9, 0, 30, 2, 2, 11], np.int32)
    sf, se = _d().plan_replicas(dev(c), 5)
    ws, ss = _d().place_replicas(dev(w), dev(s), se)
    se_h = host(se)
    assert np.array_equal(host(ws), w[se_h])
    assert np.array_equal(host(ss).view(np.uint32), s[se_h].view(np.uint32))
