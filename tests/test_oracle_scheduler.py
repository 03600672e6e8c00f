"""Pins for the batch planner oracle.

* brute force: the DP cost equals the minimum over ALL set partitions and the
  DP plan equals the best contiguous plan (with its tie-break) for n <= 8;
* closed forms: c = 0 gives zero padding; equal lengths give the fewest
  batches; a huge overhead gives one batch when it fits;
* hand-worked examples in tests/golden/hand_examples.json.

The measured-cost planner (cost of a batch = a table entry C[|B|, max_len])
has the same three kinds of pins: brute force over all set partitions and
all contiguous plans for random length-monotone tables, a constant table
(cost = number of batches, closed form), and hand-worked examples.
"""
import json
import os

import numpy as np
import pytest

import oracle
from oracle import (best_contiguous_plan, exhaustive_set_partition_cost, pack_offsets,
                    plan_batches, plan_cost)

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def test_dp_equals_exhaustive_search():
    rng = np.random.default_rng(2024)
    n_cases = 0
    for _ in range(400):
        n = int(rng.integers(1, 9))
        T = int(rng.choice([8, 12, 16, 24, 40]))
        c = int(rng.choice([0, 1, 3, 8, 20]))
        hi = int(rng.choice([3, 6, T]))                    # small hi -> many ties
        lengths = rng.integers(1, min(hi, T) + 1, size=n)
        order, starts, cost = plan_batches(lengths, T, c)
        assert cost == exhaustive_set_partition_cost(lengths, T, c)
        best_starts, best_cost = best_contiguous_plan(lengths, T, c)
        assert best_cost == cost
        assert list(starts) == best_starts
        assert plan_cost(lengths, order, list(starts), c) == cost
        n_cases += 1
    assert n_cases == 400


def test_plan_is_valid_partition_within_budget():
    rng = np.random.default_rng(7)
    lengths = rng.integers(2, 101, size=500)
    order, starts, cost = plan_batches(lengths, 4096, 1024)
    assert sorted(order.tolist()) == list(range(500))
    assert starts[0] == 0 and starts[-1] == 500 and np.all(np.diff(starts) > 0)
    s = lengths[order]
    assert np.all(np.diff(s) >= 0)
    for a, b in zip(starts[:-1], starts[1:]):
        assert (b - a) * s[b - 1] <= 4096
    assert plan_cost(lengths, order, list(starts), 1024) == cost


def test_zero_overhead_means_zero_padding():
    rng = np.random.default_rng(3)
    for _ in range(50):
        lengths = rng.integers(1, 9, size=int(rng.integers(1, 40)))
        _, _, cost = plan_batches(lengths, 16, 0)
        assert cost == int(lengths.sum())


def test_equal_lengths_fewest_batches():
    for n, ell, T in [(10, 3, 9), (7, 5, 5), (64, 128, 16384), (2000, 51, 4096)]:
        _, starts, cost = plan_batches([ell] * n, T, 7)
        nb = -(-n // (T // ell))
        assert len(starts) - 1 == nb
        assert cost == nb * 7 + n * ell


def test_huge_overhead_gives_one_batch_when_it_fits():
    lengths = [3, 9, 1, 4, 4, 7]
    _, starts, cost = plan_batches(lengths, 6 * 9, 10 ** 6)
    assert list(starts) == [0, 6]
    assert cost == 10 ** 6 + 6 * 9


def test_hand_examples():
    with open(os.path.join(GOLD, "hand_examples.json")) as f:
        cases = json.load(f)["scheduler"]
    for c in cases:
        order, starts, cost = plan_batches(c["lengths"], c["max_tokens"], c["overhead"])
        assert order.tolist() == c["order"]
        assert starts.tolist() == c["batch_starts"]
        assert cost == c["total_cost"]


def test_stable_sort_on_ties():
    order, _, _ = plan_batches([3, 1, 3, 1, 3], 100, 5)
    assert order.tolist() == [1, 3, 0, 2, 4]


def test_invalid_inputs_raise():
    with pytest.raises(ValueError):
        plan_batches([0, 3], 10, 1)
    with pytest.raises(ValueError):
        plan_batches([11], 10, 1)
    with pytest.raises(ValueError):
        plan_batches([1], 10, -1)


def test_empty_request_list():
    order, starts, cost = plan_batches([], 10, 1)
    assert order.size == 0 and starts.tolist() == [0] and cost == 0


def test_pack_offsets_prefix_sums():
    lengths = np.array([5, 1, 3, 3, 8])
    order = [1, 2, 3, 0, 4]
    assert pack_offsets(lengths, order, 0, 3).tolist() == [0, 1, 4, 7]
    assert pack_offsets(lengths, order, 3, 5).tolist() == [0, 5, 13]
    assert pack_offsets(lengths, order, 2, 2).tolist() == [0]


# ------------------------------------------------------ measured cost table

def random_monotone_table(rng, max_batch, max_len):
    """Random integer table, non-decreasing along the length (a row per batch
    size), with steps of 0 often enough to create ties."""
    steps = rng.integers(0, 4, size=(max_batch, max_len)) * (rng.random((max_batch, max_len)) < 0.7)
    return np.cumsum(steps, axis=1) + rng.integers(0, 5, size=(max_batch, 1))


def test_table_dp_equals_exhaustive_search():
    """Brute force over ALL set partitions (optimal cost) and over all
    contiguous plans of the sorted order (plan and tie-break)."""
    rng = np.random.default_rng(77)
    for _ in range(300):
        n = int(rng.integers(1, 8))
        max_len = int(rng.choice([3, 6, 10]))
        max_batch = int(rng.integers(1, 6))
        T = int(rng.choice([max_len, 2 * max_len, 40]))
        table = random_monotone_table(rng, max_batch, max_len)
        lengths = rng.integers(1, max_len + 1, size=n)
        order, starts, cost = oracle.plan_batches_table(lengths, T, table)
        assert cost == oracle.exhaustive_set_partition_cost_table(lengths, T, table)
        best_starts, best_cost = oracle.best_contiguous_plan_table(lengths, T, table)
        assert (list(starts), cost) == (best_starts, best_cost)
        assert oracle.plan_cost_table(lengths, order, list(starts), table) == cost
        sizes = np.diff(starts)
        assert np.all(sizes <= max_batch)
        assert np.all(sizes * lengths[order][starts[1:] - 1] <= T)


def test_table_hand_examples():
    with open(os.path.join(GOLD, "hand_examples.json")) as f:
        cases = json.load(f)["scheduler_table"]
    for c in cases:
        order, starts, cost = oracle.plan_batches_table(c["lengths"], c["max_tokens"], c["table"])
        assert order.tolist() == c["order"]
        assert starts.tolist() == c["batch_starts"]
        assert cost == c["total_cost"]


def test_table_constant_cost_counts_batches():
    """C = 1 everywhere: the cost is the number of batches, so equal lengths
    give ceil(n / min(max_batch, T // len)) batches."""
    for n, ell, T, mb in [(10, 3, 9, 5), (10, 3, 100, 4), (1, 7, 7, 1), (33, 2, 64, 8)]:
        table = np.ones((mb, ell), dtype=np.int64)
        _, starts, cost = oracle.plan_batches_table([ell] * n, T, table)
        k = min(mb, T // ell)
        assert cost == len(starts) - 1 == -(-n // k)


def test_table_rejects_bad_tables():
    with pytest.raises(ValueError):
        oracle.plan_batches_table([1, 2], 10, [[1, 0, 2]])        # falls along the length
    with pytest.raises(ValueError):
        oracle.plan_batches_table([1, 2], 10, [[-1, 0]])          # negative
    with pytest.raises(ValueError):
        oracle.plan_batches_table([3], 10, [[1, 2]])              # length beyond the table
    order, starts, cost = oracle.plan_batches_table([], 10, [[1]])
    assert order.size == 0 and starts.tolist() == [0] and cost == 0
