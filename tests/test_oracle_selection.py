"""Pins for the best-of-N selection oracle ("Learning to summarize from human
feedback", Method adaptation: keep the candidate the reward model scores
highest; equal rewards resolve to the lowest index -- the reading used)."""
import json
import os

import numpy as np
import pytest

import oracle

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "hand_examples.json")))


@pytest.mark.parametrize("case", GOLDEN["best_of_n"], ids=lambda c: c["derivation"][:30])
def test_hand_examples(case):
    assert oracle.best_of_n(case["rewards"], case["counts"]) == case["best"]


def test_distinct_rewards_match_numpy_argmax_per_prompt():
    rng = np.random.default_rng(5)
    for _ in range(50):
        counts = rng.integers(1, 9, size=rng.integers(1, 12))
        r = rng.standard_normal(int(counts.sum()))
        starts = np.concatenate([[0], np.cumsum(counts)])
        want = [int(np.argmax(r[a:b])) for a, b in zip(starts[:-1], starts[1:])]
        assert oracle.best_of_n(r.tolist(), counts.tolist()) == want


def test_ties_on_small_integers_brute_force():
    """Brute force over every reward vector in {0,1,2}^4: the answer is the
    first position holding the maximum."""
    import itertools
    for r in itertools.product([0, 1, 2], repeat=4):
        m = max(r)
        assert oracle.best_of_n(list(r), [4]) == [r.index(m)]


def test_moving_the_maximum_moves_the_answer():
    base = [0.0] * 7
    for k in range(7):
        r = list(base)
        r[k] = 1.0
        assert oracle.best_of_n(r, [7]) == [k]


def test_bad_counts_raise():
    with pytest.raises(ValueError):
        oracle.best_of_n([1.0, 2.0], [0, 2])
    with pytest.raises(ValueError):
        oracle.best_of_n([1.0, 2.0], [3])
    with pytest.raises(ValueError):
        oracle.best_of_n([1.0, 2.0, 3.0], [2])
