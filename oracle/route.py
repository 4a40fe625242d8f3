"""Auxiliary-loss-free, group-limited top-K routing and the token permute.

Sources:
* V3 notes §4: each expert i keeps a bias b_i; the top-K choice is made on
  the corrected affinity s_{i,t} + b_i while the gating weight of a chosen
  expert comes from the raw s_{i,t} (the formulas themselves were lost from
  the page; only this prose survives).
* V3 notes §2: 256 routed experts, 8 chosen per token, plus one shared expert;
  only the chosen experts' gates are non-zero.
* V3 notes §4.2 and the infra answer (group-routing paragraph): routing is
  node-limited, a token reaches experts on at most 4 nodes; the training run
  spreads the experts over 8 nodes.  No token is dropped.

Readings taken where the pages are silent or garbled:
* affinity is the sigmoid, s = fl32(1 / (1 + exp(-z))) evaluated in float64
  and rounded once to float32;
* key = fl32(s + b) (float32 addition);
* the E experts form G contiguous groups of E/G ("nodes"); a group's score is
  the float32 sum, in descending order, of its ceil(K/Mg) largest keys; the Mg
  best groups are kept under the order (score descending, group index
  ascending);
* among the experts of the kept groups the K best under (key descending,
  expert index ascending) are chosen and listed in that order;
* gate_k = s_k / sum of s over the chosen experts (no further scale factor);
* the permute lists, expert by expert in ascending expert order, the tokens
  that chose it in ascending token order; inv maps (token, k) to that row.
"""

import numpy as np


def affinity(logits: np.ndarray) -> np.ndarray:
    """s = fl32(sigmoid(z)), sigmoid evaluated in float64."""
    z = np.asarray(logits, dtype=np.float32).astype(np.float64)
    return (1.0 / (1.0 + np.exp(-z))).astype(np.float32)


def keys(s: np.ndarray, bias: np.ndarray) -> np.ndarray:
    """Selection key s + b, rounded to float32."""
    return (np.asarray(s, np.float32) + np.asarray(bias, np.float32)[None, :]).astype(np.float32)


def group_scores(key: np.ndarray, n_groups: int, n_top: int) -> np.ndarray:
    """score[t][g] = float32 sum (largest first) of the n_top largest keys of
    group g = experts [g*E/G, (g+1)*E/G)."""
    t, e = key.shape
    grp = key.reshape(t, n_groups, e // n_groups)
    top = -np.sort(-grp, axis=2)[:, :, :n_top]               # descending
    acc = top[:, :, 0].astype(np.float32)
    for i in range(1, n_top):
        acc = (acc + top[:, :, i]).astype(np.float32)
    return acc


def route(logits, bias, n_groups: int, groups_kept: int, top_k: int):
    """Routing of T tokens.

    logits float32 [T][E], bias float32 [E].
    Returns dict with topk_idx int32 [T][K], gates float64 [T][K],
    s float32 [T][E], key float32 [T][E], group_score float32 [T][G],
    chosen_groups int32 [T][Mg].
    """
    logits = np.asarray(logits, dtype=np.float32)
    t, e = logits.shape
    per_group = e // n_groups
    n_top = -(-top_k // groups_kept)                           # ceil(K / Mg)

    s = affinity(logits)
    key = keys(s, bias)
    score = group_scores(key, n_groups, n_top)

    # stable sort of the negated values = (value desc, index asc)
    chosen_groups = np.argsort(-score, axis=1, kind="stable")[:, :groups_kept]

    allowed = np.zeros((t, n_groups), dtype=bool)
    np.put_along_axis(allowed, chosen_groups, True, axis=1)
    allowed_e = np.repeat(allowed, per_group, axis=1)
    masked = np.where(allowed_e, key, -np.inf)
    topk_idx = np.argsort(-masked, axis=1, kind="stable")[:, :top_k].astype(np.int32)

    s_sel = np.take_along_axis(s, topk_idx, axis=1).astype(np.float64)
    gates = s_sel / s_sel.sum(axis=1, keepdims=True) if t else s_sel

    return {
        "topk_idx": topk_idx,
        "gates": gates,
        "s": s,
        "key": key,
        "group_score": score,
        "chosen_groups": chosen_groups.astype(np.int32),
    }


def permute(topk_idx: np.ndarray, n_experts: int):
    """counts int32 [E], offsets int32 [E+1], perm int32 [T*K] (row -> token),
    inv int32 [T][K] ((token, k) -> row).  Rows are grouped by expert in
    ascending expert order and, within an expert, by ascending token."""
    topk_idx = np.asarray(topk_idx, dtype=np.int64)
    t, k = topk_idx.shape
    e_flat = topk_idx.reshape(-1)
    t_flat = np.repeat(np.arange(t, dtype=np.int64), k)
    counts = np.bincount(e_flat, minlength=n_experts).astype(np.int32)
    offsets = np.zeros(n_experts + 1, dtype=np.int32)
    offsets[1:] = np.cumsum(counts)
    order = np.lexsort((t_flat, e_flat))                       # expert, then token
    perm = t_flat[order].astype(np.int32)
    inv_flat = np.empty(t * k, dtype=np.int32)
    inv_flat[order] = np.arange(t * k, dtype=np.int32)
    return counts, offsets, perm, inv_flat.reshape(t, k)
