"""Decode-serving bookkeeping: redundant replicas of hot experts and the rule
that spreads an expert's tokens over its replicas.

Test infrastructure: imported only by the tests, the smoke check and the
benchmark's CPU baseline; the library never uses it.

Sources: V3 notes §8 (the deployment section, prefill and decode designed
apart): in decode the shared expert counts as a routed expert that every
token takes, so a token uses 9 experts; some GPUs hold the shared expert and
redundant experts; the experts that run hot in the live traffic are copied
periodically, from statistics gathered online, and the placement adjusted.
Infra answer, inference paragraph: decode runs 320-way expert parallelism,
256 experts plus 64 copies of hot ones.

The pages fix neither how many copies each hot expert gets nor how a token
picks a copy.  The readings taken here:

* ``plan_replicas``: R extra slots go one at a time to the expert with the
  largest load per slot, c_e / n_e (compared exactly, as c_a n_b vs c_b n_a),
  the lowest index winning ties.  Every expert keeps at least one slot, and an
  expert's slots are consecutive: slot_first[e] = sum of n_f over f < e.
  This greedy rule minimises max_e c_e / n_e over all n >= 1 with
  sum n = E + R (the pins check it by brute force).
* ``physical_offsets``: the rows of expert e (tokens ascending, as the
  permute orders them) are cut into n_e contiguous chunks, chunk j starting at
  row offsets[e] + floor(j c_e / n_e), so sibling chunks differ by at most
  one row and the permutation itself is unchanged.
* The layer output does not depend on the plan: every row is computed from
  the same expert weights whichever copy holds it.  oracle.layer is the
  oracle for the output.
"""

import numpy as np


def plan_replicas(counts, n_extra: int):
    """counts [E] (non-negative int) -> (n_rep [E], slot_first [E+1],
    slot_expert [E + n_extra]), all int64."""
    c = [int(v) for v in np.asarray(counts).reshape(-1)]
    if any(v < 0 for v in c):
        raise ValueError("counts must be non-negative")
    if n_extra < 0:
        raise ValueError("n_extra must be non-negative")
    n = [1] * len(c)
    for _ in range(n_extra):
        best = 0
        for e in range(1, len(c)):
            # c[e] / n[e] > c[best] / n[best], exactly; ties keep the lower index
            if c[e] * n[best] > c[best] * n[e]:
                best = e
        n[best] += 1
    n_rep = np.array(n, dtype=np.int64)
    slot_first = np.concatenate([[0], np.cumsum(n_rep)]).astype(np.int64)
    slot_expert = np.repeat(np.arange(len(c), dtype=np.int64), n_rep)
    return n_rep, slot_first, slot_expert


def max_load_per_slot(counts, n_rep) -> float:
    """max over experts of counts[e] / n_rep[e]."""
    c = np.asarray(counts, dtype=np.float64)
    return float(np.max(c / np.asarray(n_rep, dtype=np.float64))) if c.size else 0.0


def physical_offsets(offsets, slot_first):
    """Group offsets [E+1] of the experts -> offsets [S+1] of the slots."""
    off = [int(v) for v in np.asarray(offsets).reshape(-1)]
    sf = [int(v) for v in np.asarray(slot_first).reshape(-1)]
    E = len(off) - 1
    if len(sf) != E + 1:
        raise ValueError("slot_first must have E+1 entries")
    out = []
    for e in range(E):
        cnt = off[e + 1] - off[e]
        ne = sf[e + 1] - sf[e]
        for j in range(ne):
            out.append(off[e] + (j * cnt) // ne)
    out.append(off[E])
    return np.array(out, dtype=np.int64)


__all__ = ["plan_replicas", "max_load_per_slot", "physical_offsets"]
