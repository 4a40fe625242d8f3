"""Pins of the oracle's routing, permute and bias update.

* hand-worked tokens (tests/golden/routing_c1.json, bias_update.json);
* brute force: among all Mg-subsets of groups and all K-subsets of allowed
  experts exactly one dominates (each member outranks each non-member under
  the stated total order); it must be the oracle's choice;
* a plain Python sort for the ungrouped special case;
* invariants: gates sum to 1, at most Mg groups and K distinct experts per
  token, counts sum to T*K, perm/inv are inverse bijections ordered by
  (expert, token).
"""

import itertools

import numpy as np
import pytest

from oracle import bias as obias
from oracle import route


def _golden_logits(g):
    E = g["E"]
    z = np.full((len(g["tokens"]), E), g["logits_default"], np.float32)
    for t, tok in enumerate(g["tokens"]):
        for k, v in tok["logits"].items():
            if k == "all":
                z[t, :] = v
            else:
                z[t, int(k)] = v
    b = np.zeros(E, np.float32)
    for k, v in g["bias_nonzero"].items():
        b[int(k)] = v
    return z, b


def test_golden_routing(golden):
    g = golden("routing_c1.json")
    z, b = _golden_logits(g)
    r = route.route(z, b, g["G"], g["Mg"], g["K"])
    for t, tok in enumerate(g["tokens"]):
        assert list(r["topk_idx"][t]) == tok["topk_idx"], t
        assert np.allclose(r["gates"][t], tok["gates"], atol=1e-6, rtol=0), t
    counts, offsets, perm, inv = route.permute(r["topk_idx"], g["E"])
    assert list(counts) == g["counts"]
    assert list(offsets) == g["offsets"]
    assert list(perm) == g["perm"]
    assert inv.tolist() == g["inv"]
    r0 = route.route(z[:1], np.zeros_like(b), g["G"], g["Mg"], g["K"])
    assert list(r0["topk_idx"][0]) == g["without_bias_token0"]["topk_idx"]
    assert np.allclose(r0["gates"][0], g["without_bias_token0"]["gates"], atol=1e-6, rtol=0)


def test_golden_bias_update(golden):
    gr = golden("routing_c1.json")
    gb = golden("bias_update.json")
    z, b = _golden_logits(gr)
    r = route.route(z, b, gr["G"], gr["Mg"], gr["K"])
    counts, *_ = route.permute(r["topk_idx"], gr["E"])
    b2 = obias.update_bias(b, counts, n_tokens=4, top_k=2, gamma=gb["gamma"])
    step = np.float32(gb["gamma"])
    want = (b + step * np.array(gb["direction"], np.float32)).astype(np.float32)
    assert np.array_equal(b2, want)
    r2 = route.route(z[2:3], b2, gr["G"], gr["Mg"], gr["K"])
    assert list(r2["topk_idx"][0]) == gb["rerouted_token2_topk_idx"]


def test_bias_update_uniform_load_is_unchanged_and_sign_zero():
    b = np.linspace(-0.01, 0.01, 8).astype(np.float32)
    counts = np.full(8, 3, np.int32)                  # T*K = 12, E*c = 24 -> down
    assert np.all(obias.update_bias(b, counts, 6, 2) < b)
    counts = np.full(8, 3, np.int32)                  # T*K = 24 = E*c -> unchanged
    assert np.array_equal(obias.update_bias(b, counts, 12, 2), b)


def _outranks(va, ia, vb, ib):
    return va > vb or (va == vb and ia < ib)


def _dominating_subsets(values, candidates, size):
    out = []
    for sub in itertools.combinations(candidates, size):
        rest = [c for c in candidates if c not in sub]
        if all(_outranks(values[a], a, values[b], b) for a in sub for b in rest):
            out.append(set(sub))
    return out


def _brute_route(key_row, n_groups, groups_kept, top_k):
    e = key_row.shape[0]
    per = e // n_groups
    n_top = -(-top_k // groups_kept)
    scores = []
    for g in range(n_groups):
        ks = [key_row[g * per + i] for i in range(per)]
        best = None
        for sub in itertools.combinations(range(per), n_top):
            vals = sorted((ks[i] for i in sub), reverse=True)
            acc = np.float32(vals[0])
            for v in vals[1:]:
                acc = np.float32(acc + np.float32(v))
            best = acc if best is None or acc > best else best
        scores.append(best)
    gsets = _dominating_subsets(scores, list(range(n_groups)), groups_kept)
    assert len(gsets) == 1
    allowed = [x for g in sorted(gsets[0]) for x in range(g * per, (g + 1) * per)]
    esets = _dominating_subsets(key_row, allowed, top_k)
    assert len(esets) == 1
    chosen = sorted(esets[0], key=lambda x: (-key_row[x], x))
    return gsets[0], chosen


@pytest.mark.parametrize("E,G,Mg,K", [(12, 4, 2, 3), (8, 2, 1, 2), (16, 4, 2, 2), (9, 3, 3, 4)])
def test_routing_matches_brute_force(E, G, Mg, K):
    r = np.random.default_rng(E * 100 + K)
    T = 200
    # few distinct values -> many exact ties in keys and group scores
    z = r.choice(np.array([-1.0, 0.0, 0.5, 1.0], np.float32), size=(T, E))
    b = r.choice(np.array([0.0, 0.0, 0.125, -0.125], np.float32), size=E)
    out = route.route(z, b, G, Mg, K)
    for t in range(T):
        gset, chosen = _brute_route(out["key"][t], G, Mg, K)
        assert set(out["chosen_groups"][t].tolist()) == gset
        assert out["topk_idx"][t].tolist() == chosen


def test_ungrouped_special_case_is_a_plain_sort():
    r = np.random.default_rng(5)
    z = r.choice(np.array([-2.0, 0.0, 0.3, 2.0], np.float32), size=(50, 32))
    out = route.route(z, np.zeros(32, np.float32), 1, 1, 6)
    s = out["s"]
    for t in range(50):
        want = sorted(range(32), key=lambda e: (-float(s[t, e]), e))[:6]
        assert out["topk_idx"][t].tolist() == want


def test_sigmoid_rounding_is_single_float32_rounding():
    z = np.array([[0.0, 2.0, -3.0, 30.0, -30.0, -104.0]], np.float32)
    s = route.affinity(z)
    import math
    want = [np.float32(1.0 / (1.0 + math.exp(-float(v)))) for v in z[0]]
    assert list(s[0]) == want
    assert s[0, 0] == 0.5


def test_routing_invariants_v3_geometry():
    r = np.random.default_rng(11)
    T, E, G, Mg, K = 512, 256, 8, 4, 8
    z = (r.standard_normal((T, E)) * 0.5).astype(np.float32)
    b = r.uniform(-0.01, 0.01, E).astype(np.float32)
    out = route.route(z, b, G, Mg, K)
    idx = out["topk_idx"]
    assert np.allclose(out["gates"].sum(axis=1), 1.0, atol=1e-12)
    assert np.all(out["gates"] > 0)
    for t in range(T):
        assert len(set(idx[t].tolist())) == K
        assert len(set((idx[t] // (E // G)).tolist())) <= Mg
        keys_t = out["key"][t][idx[t]]
        assert np.all(keys_t[:-1] >= keys_t[1:])
    counts, offsets, perm, inv = route.permute(idx, E)
    assert counts.sum() == T * K and offsets[-1] == T * K and offsets[0] == 0
    assert sorted(inv.reshape(-1).tolist()) == list(range(T * K))
    for t in range(T):
        for k in range(K):
            row = inv[t, k]
            e = idx[t, k]
            assert perm[row] == t
            assert offsets[e] <= row < offsets[e + 1]
    for e in range(E):
        seg = perm[offsets[e]:offsets[e + 1]]
        assert np.all(np.diff(seg) > 0)


def test_empty_batch():
    out = route.route(np.zeros((0, 16), np.float32), np.zeros(16, np.float32), 4, 2, 2)
    counts, offsets, perm, inv = route.permute(out["topk_idx"], 16)
    assert counts.sum() == 0 and offsets[-1] == 0 and perm.size == 0 and inv.shape == (0, 2)
