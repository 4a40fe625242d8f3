"""Pins of oracle.serving (V3 notes §8: redundant copies of hot experts,
chosen from observed loads; the shared expert as a 9th routed expert)."""

import itertools
from fractions import Fraction

import numpy as np
import pytest

from oracle import serving as osv


def _compositions(total, parts):
    """Every n with n_e >= 1 and sum n = total."""
    for cut in itertools.combinations(range(1, total), parts - 1):
        edges = (0,) + cut + (total,)
        yield [edges[i + 1] - edges[i] for i in range(parts)]


def _max_ratio(c, n):
    return max(Fraction(ci, ni) for ci, ni in zip(c, n))


@pytest.mark.parametrize("seed", range(40))
def test_greedy_plan_is_optimal_by_brute_force(seed):
    """No distribution of the extra slots gives a smaller maximum load per slot."""
    r = np.random.default_rng(seed)
    E = int(r.integers(1, 5))
    R = int(r.integers(0, 6))
    c = [int(v) for v in r.integers(0, 30, E)]
    n_rep, _, _ = osv.plan_replicas(c, R)
    assert n_rep.sum() == E + R and n_rep.min() >= 1
    best = min(_max_ratio(c, n) for n in _compositions(E + R, E))
    assert _max_ratio(c, n_rep) == best, (c, R, n_rep.tolist())


def test_hand_worked_plan_and_offsets():
    # loads 10, 3, 6, 0 and three extra slots:
    #   10/1 largest -> expert 0 (n0 = 2, load 5)
    #   6/1 largest  -> expert 2 (n2 = 2, load 3)
    #   5 largest    -> expert 0 (n0 = 3, load 10/3)
    n_rep, slot_first, slot_expert = osv.plan_replicas([10, 3, 6, 0], 3)
    assert n_rep.tolist() == [3, 1, 2, 1]
    assert slot_first.tolist() == [0, 3, 4, 6, 7]
    assert slot_expert.tolist() == [0, 0, 0, 1, 2, 2, 3]
    # rows: expert 0 -> 0..9, expert 1 -> 10..12, expert 2 -> 13..18, expert 3 none
    phys = osv.physical_offsets([0, 10, 13, 19, 19], slot_first)
    # expert 0 in 3 chunks: starts 0, floor(10/3) = 3, floor(20/3) = 6 -> sizes 3, 3, 4
    assert phys.tolist() == [0, 3, 6, 10, 13, 16, 19, 19]


def test_ties_go_to_the_lowest_index():
    assert osv.plan_replicas([4, 4], 1)[0].tolist() == [2, 1]
    assert osv.plan_replicas([3, 6, 6], 1)[0].tolist() == [1, 2, 1]
    # after two extra slots (to experts 1 and 2) all three loads are 3: expert 0 wins the third
    assert osv.plan_replicas([3, 6, 6], 3)[0].tolist() == [2, 2, 2]
    # all idle: expert 0 takes every extra slot
    assert osv.plan_replicas([0, 0, 0], 2)[0].tolist() == [3, 1, 1]


def test_no_extra_slots_is_the_identity():
    c = np.random.default_rng(1).integers(0, 50, 256)
    n_rep, slot_first, slot_expert = osv.plan_replicas(c, 0)
    assert np.all(n_rep == 1) and slot_first.tolist() == list(range(257))
    off = np.concatenate([[0], np.cumsum(c)])
    assert np.array_equal(osv.physical_offsets(off, slot_first), off)


def test_physical_offsets_invariants_on_a_skewed_load():
    r = np.random.default_rng(2)
    p = 1.0 / np.arange(1, 257) ** 1.1
    c = np.bincount(r.choice(256, size=64 * 8, p=p / p.sum()), minlength=256)
    n_rep, slot_first, slot_expert = osv.plan_replicas(c, 32)
    off = np.concatenate([[0], np.cumsum(c)])
    phys = osv.physical_offsets(off, slot_first)
    assert len(phys) == 256 + 32 + 1 and phys[0] == 0 and phys[-1] == off[-1]
    assert np.all(np.diff(phys) >= 0)
    for e in range(256):
        sizes = np.diff(phys[slot_first[e]:slot_first[e + 1] + 1])
        assert sizes.sum() == c[e] and sizes.max() - sizes.min() <= 1
        assert phys[slot_first[e]] == off[e]
    # the copies halve (at least) the hottest expert's load per slot
    assert osv.max_load_per_slot(c, n_rep) <= c.max() / 2


def test_rejects_bad_input():
    with pytest.raises(ValueError):
        osv.plan_replicas([1, -1], 1)
    with pytest.raises(ValueError):
        osv.plan_replicas([1, 1], -1)
    with pytest.raises(ValueError):
        osv.physical_offsets([0, 1, 2], [0, 1])
