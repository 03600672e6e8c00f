"""Pins of oracle/memplan.py (arena placement of tensors with lifetimes).

The pages give no algorithm or worked example for the allocator, so the
oracle is pinned by what placement itself fixes: closed forms (lifetimes all
disjoint -> the largest tensor; all meeting -> the sum), the lower bound (the
bytes alive at one step) met by the brute-force optimum on interval chains,
touching intervals (steps are inclusive), alignment, and an exhaustive check
that the brute force never beats the lower bound and never loses to greedy.
"""
import itertools

import numpy as np
import pytest

from oracle import memplan as mp


def test_disjoint_lifetimes_share_everything():
    nb, f, l = [100, 300, 200], [0, 2, 4], [1, 3, 5]
    off, total = mp.greedy_by_size(nb, f, l)
    assert off == [0, 0, 0] and total == 300
    assert mp.optimum(nb, f, l) == 300 == mp.lower_bound(nb, f, l)


def test_meeting_lifetimes_share_nothing():
    nb, f, l = [100, 300, 200], [0, 0, 1], [5, 2, 3]
    off, total = mp.greedy_by_size(nb, f, l)
    assert total == 600 and mp.valid(nb, f, l, off)
    assert sorted(off) == [0, 300, 500]          # largest first, then 200, then 100


def test_touching_intervals_meet():
    # [0,2] and [2,4] share step 2: they may not share bytes
    nb, f, l = [64, 64], [0, 2], [2, 4]
    off, total = mp.greedy_by_size(nb, f, l)
    assert total == 128 and mp.valid(nb, f, l, off)
    assert not mp.valid(nb, f, l, [0, 0])
    assert mp.valid([64, 64], [0, 3], [2, 4], [0, 0])


def test_gap_reuse_and_alignment():
    # a (0..2) 100 B and c (4..6) 50 B both meet b (1..5): b stacks above the larger one
    nb, f, l = [100, 120, 50], [0, 1, 4], [2, 5, 6]
    off, total = mp.greedy_by_size(nb, f, l)
    assert off == [120, 0, 120] and total == 220
    off, total = mp.greedy_by_size(nb, f, l, align=64)
    assert off == [128, 0, 128] and total == 256
    assert all(o % 64 == 0 for o in off)


def test_zero_sized_records_take_no_room():
    nb, f, l = [0, 40, 0], [0, 0, 0], [9, 9, 9]
    off, total = mp.greedy_by_size(nb, f, l)
    assert total == 40 and off == [0, 0, 0]


def test_chain_meets_lower_bound():
    # a path of intervals: alive sets are consecutive pairs
    nb = [30, 70, 20, 90, 10]
    f = [0, 1, 2, 3, 4]
    l = [1, 2, 3, 4, 5]
    lb = mp.lower_bound(nb, f, l)
    assert lb == 110                                   # 20 + 90 at step 3
    assert mp.optimum(nb, f, l) == lb
    off, total = mp.greedy_by_size(nb, f, l)
    assert mp.valid(nb, f, l, off) and total == lb


def test_brute_force_between_bound_and_greedy():
    rng = np.random.default_rng(5)
    for _ in range(150):
        n = int(rng.integers(1, 7))
        nb = [int(x) for x in rng.integers(0, 9, size=n) * 16]
        f = [int(x) for x in rng.integers(0, 6, size=n)]
        l = [a + int(rng.integers(0, 4)) for a in f]
        opt = mp.optimum(nb, f, l)
        off, g = mp.greedy_by_size(nb, f, l)
        assert mp.valid(nb, f, l, off)
        assert mp.lower_bound(nb, f, l) <= opt <= g


def test_lowest_fit_places_at_the_smallest_free_offset():
    rng = np.random.default_rng(8)
    for _ in range(100):
        n = int(rng.integers(2, 6))
        nb = [int(x) for x in rng.integers(1, 6, size=n)]
        f = [int(x) for x in rng.integers(0, 4, size=n)]
        l = [a + int(rng.integers(0, 3)) for a in f]
        order = list(rng.permutation(n))
        off = mp.lowest_fit(nb, f, l, order)
        for k, i in enumerate(order):
            # no smaller offset would have been free of the records placed before it
            earlier = [j for j in order[:k] if mp.meets(f[i], l[i], f[j], l[j])]
            for c in range(off[i]):
                clash = any(c < off[j] + nb[j] and off[j] < c + nb[i] for j in earlier)
                assert clash, (nb, f, l, order, i, c)


def test_exhaustive_small_cases_against_set_enumeration():
    # n = 3, unit steps: optimum equals the best over all offset assignments
    # on a small grid (independent of the order-based search)
    nb, f, l = [2, 3, 1], [0, 1, 0], [1, 2, 2]
    best = None
    for offs in itertools.product(range(7), repeat=3):
        if mp.valid(nb, f, l, list(offs)):
            size = mp.arena_size(nb, list(offs))
            best = size if best is None else min(best, size)
    assert mp.optimum(nb, f, l) == best
