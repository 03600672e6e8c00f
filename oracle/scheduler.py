"""Batch planner oracle: length-sorted dynamic program plus exhaustive checks.

TurboTransformers review (Abstract; Proposed method): requests of variable
length are sorted by length and grouped by a dynamic-programming batch
scheduler so that padding is minimal and throughput optimal.  The page gives
no cost formula; the reading used here is

    cost(plan) = sum over batches B of ( c + |B| * max_len(B) ),
    subject to  |B| * max_len(B) <= T  for every batch,

i.e. the padded token count of each batch plus a fixed per-batch overhead c,
under a padded-token budget T.  With this budget an exchange argument shows
that some optimal partition is contiguous in sorted order, so the DP over
sorted prefixes is optimal over all set partitions; the exhaustive searches
below check exactly that on small inputs.

Ties: requests sort by (length, index); the DP scans split points in
ascending order and keeps the first minimum, so among optimal plans it
returns the one whose batch-start list, read from the last batch backwards,
is lexicographically smallest.
"""
import itertools

import numpy as np


def _check(lengths, max_tokens, overhead):
    lengths = [int(v) for v in lengths]
    if overhead < 0:
        raise ValueError("batch overhead must be >= 0")
    for v in lengths:
        if v < 1 or v > max_tokens:
            raise ValueError(f"length {v} outside [1, {max_tokens}]")
    return lengths


def sort_order(lengths):
    """Indices sorted by (length, original index)."""
    return sorted(range(len(lengths)), key=lambda i: (int(lengths[i]), i))


def plan_batches(lengths, max_tokens, overhead):
    """DP plan -> (order int32[n], batch_starts int32[B+1], total_cost int).

    f[0] = 0;  f[i] = min over j < i with (i-j)*s[i-1] <= T of
    f[j] + c + (i-j)*s[i-1], where s are the sorted lengths (the batch
    [j, i) has its longest request last).  The first minimising j is kept.
    """
    lengths = _check(lengths, max_tokens, overhead)
    n = len(lengths)
    order = sort_order(lengths)
    s = np.array([lengths[i] for i in order], dtype=np.int64)
    f = np.zeros(n + 1, dtype=np.int64)
    arg = np.zeros(n + 1, dtype=np.int64)
    for i in range(1, n + 1):
        j = np.arange(i, dtype=np.int64)
        size = i - j
        cost = f[:i] + overhead + size * s[i - 1]
        cost = np.where(size * s[i - 1] <= max_tokens, cost, np.iinfo(np.int64).max)
        k = int(np.argmin(cost))          # first minimum = smallest j
        f[i], arg[i] = cost[k], k
    starts = [n]
    while starts[-1] > 0:
        starts.append(int(arg[starts[-1]]))
    starts.reverse()
    if n == 0:
        starts = [0]
    return (np.array(order, dtype=np.int32), np.array(starts, dtype=np.int32), int(f[n]))


def plan_cost(lengths, order, starts, overhead):
    """Cost of a contiguous plan over ``order``: sum of c + |B| * max_len(B)."""
    total = 0
    for a, b in zip(starts[:-1], starts[1:]):
        batch = [int(lengths[order[k]]) for k in range(a, b)]
        total += overhead + len(batch) * max(batch)
    return total


def pack_offsets(lengths, order, begin, end):
    """Exclusive prefix sum of the lengths of order[begin:end] (packed layout)."""
    out = [0]
    for k in range(begin, end):
        out.append(out[-1] + int(lengths[order[k]]))
    return np.array(out, dtype=np.int32)


# ------------------------------------------------------------- brute force

def _set_partitions(n):
    """All set partitions of range(n) as restricted-growth label lists."""
    labels = [0] * n

    def rec(i, m):
        if i == n:
            yield list(labels)
            return
        for b in range(m + 1):
            labels[i] = b
            yield from rec(i + 1, m + 1 if b == m else m)

    if n == 0:
        yield []
        return
    yield from rec(1, 1)


def exhaustive_set_partition_cost(lengths, max_tokens, overhead):
    """Minimum cost over ALL set partitions (n <= 8): the true optimum."""
    lengths = _check(lengths, max_tokens, overhead)
    n = len(lengths)
    if n == 0:
        return 0
    best = None
    for lab in _set_partitions(n):
        groups = {}
        for i, g in enumerate(lab):
            groups.setdefault(g, []).append(lengths[i])
        ok, cost = True, 0
        for g in groups.values():
            pad = len(g) * max(g)
            if pad > max_tokens:
                ok = False
                break
            cost += overhead + pad
        if ok and (best is None or cost < best):
            best = cost
    return best


def best_contiguous_plan(lengths, max_tokens, overhead):
    """Enumerate all 2^(n-1) contiguous partitions of the sorted order.

    Returns (starts, cost) of the minimum-cost feasible plan, ties broken by
    the batch-start list read backwards (lexicographically smallest).
    """
    lengths = _check(lengths, max_tokens, overhead)
    n = len(lengths)
    order = sort_order(lengths)
    if n == 0:
        return [0], 0
    best = None
    for cuts in itertools.product([0, 1], repeat=n - 1):
        starts = [0] + [k + 1 for k, c in enumerate(cuts) if c] + [n]
        feasible = True
        for a, b in zip(starts[:-1], starts[1:]):
            if (b - a) * int(lengths[order[b - 1]]) > max_tokens:
                feasible = False
                break
        if not feasible:
            continue
        cost = plan_cost(lengths, order, starts, overhead)
        key = (cost, starts[::-1])
        if best is None or key < best[0]:
            best = (key, starts)
    return best[1], best[0][0]


# ------------------------------------------------------ measured cost table
#
# TurboTransformers review (Abstract; Proposed method): the batch scheduler's
# goal is throughput on variable-length requests, and the time of a batch on
# the GPU is not linear in its padded size.  Reading used for the measured
# cost model: the cost of a batch B is a table entry C[|B|, max_len(B)]
# (e.g. the measured latency of |B| sequences of that length), subject to
# |B| <= max_batch and |B| * max_len(B) <= T.  When every row of C is
# non-decreasing in the length, contiguous partitions of the sorted order are
# again optimal over all set partitions (give the j-th batch in order of
# maximum the next |B_j| requests of the sorted list: its maximum can only
# fall), so the same prefix DP applies with the table in place of c + |B| m.

def _check_table(lengths, max_tokens, table):
    table = np.asarray(table, dtype=np.int64)
    if table.ndim != 2 or table.shape[0] < 1 or table.shape[1] < 1:
        raise ValueError("cost table must be a non-empty [max_batch, max_len] array")
    if np.any(table < 0):
        raise ValueError("cost table entries must be >= 0")
    if np.any(np.diff(table, axis=1) < 0):
        raise ValueError("cost table rows must be non-decreasing in the length")
    lengths = [int(v) for v in lengths]
    for v in lengths:
        if v < 1 or v > max_tokens or v > table.shape[1]:
            raise ValueError(f"length {v} outside [1, min({max_tokens}, {table.shape[1]})]")
    return lengths, table


def table_batch_cost(table, size, max_len):
    """C[size, max_len] with 1-based size and length."""
    return int(table[size - 1, max_len - 1])


def plan_batches_table(lengths, max_tokens, table):
    """DP plan under a cost table -> (order, batch_starts, total_cost).

    f[0] = 0;  f[i] = min over j < i with i-j <= max_batch and
    (i-j)*s[i-1] <= T of  f[j] + C[i-j, s[i-1]];  first minimising j kept.
    """
    lengths, table = _check_table(lengths, max_tokens, table)
    n = len(lengths)
    max_batch = table.shape[0]
    order = sort_order(lengths)
    s = [lengths[i] for i in order]
    f = [0] * (n + 1)
    arg = [0] * (n + 1)
    for i in range(1, n + 1):
        best = None
        for j in range(i):
            size = i - j
            if size > max_batch or size * s[i - 1] > max_tokens:
                continue
            v = f[j] + table_batch_cost(table, size, s[i - 1])
            if best is None or v < best:
                best, arg[i] = v, j
        f[i] = best
    starts = [n]
    while starts[-1] > 0:
        starts.append(arg[starts[-1]])
    starts.reverse()
    return (np.array(order, dtype=np.int32), np.array(starts, dtype=np.int32), int(f[n]))


def plan_cost_table(lengths, order, starts, table):
    """Cost of a contiguous plan over ``order`` under the table."""
    total = 0
    for a, b in zip(starts[:-1], starts[1:]):
        batch = [int(lengths[order[k]]) for k in range(a, b)]
        total += table_batch_cost(table, len(batch), max(batch))
    return total


def exhaustive_set_partition_cost_table(lengths, max_tokens, table):
    """Minimum table cost over ALL set partitions (n <= 8)."""
    lengths, table = _check_table(lengths, max_tokens, table)
    n = len(lengths)
    if n == 0:
        return 0
    best = None
    for lab in _set_partitions(n):
        groups = {}
        for i, g in enumerate(lab):
            groups.setdefault(g, []).append(lengths[i])
        cost, ok = 0, True
        for g in groups.values():
            if len(g) > table.shape[0] or len(g) * max(g) > max_tokens:
                ok = False
                break
            cost += table_batch_cost(table, len(g), max(g))
        if ok and (best is None or cost < best):
            best = cost
    return best


def best_contiguous_plan_table(lengths, max_tokens, table):
    """All 2^(n-1) contiguous plans of the sorted order under the table;
    ties broken by the start list read backwards (smallest)."""
    lengths, table = _check_table(lengths, max_tokens, table)
    n = len(lengths)
    order = sort_order(lengths)
    if n == 0:
        return [0], 0
    best = None
    for cuts in itertools.product([0, 1], repeat=n - 1):
        starts = [0] + [k + 1 for k, c in enumerate(cuts) if c] + [n]
        if any((b - a) > table.shape[0] or (b - a) * lengths[order[b - 1]] > max_tokens
               for a, b in zip(starts[:-1], starts[1:])):
            continue
        key = (plan_cost_table(lengths, order, starts, table), starts[::-1])
        if best is None or key < best[0]:
            best = (key, starts)
    return best[1], best[0][0]
