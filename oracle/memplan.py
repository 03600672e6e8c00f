"""Placement of tensors with lifetimes in one memory arena (oracle; test
infrastructure only).

"TurboTransformers: An Efficient GPU Serving System For Transformer Models"
(review), Proposed method and Main results: a sequence-length-aware allocator
for variable-length inputs keeps the footprint of the intermediate tensors
low without allocating per request.  The reading used here (the pages give
no algorithm): every intermediate of a pass is a record (bytes, first step,
last step); two records may share bytes only if their step intervals are
disjoint; the arena needs the largest end offset.  The library places
records largest first (ties: lower index) at the lowest fitting offset.

Plain definitions, written for checking by eye:
  * ``rounded`` -- bytes rounded up to the alignment;
  * ``meets`` -- two closed step intervals share a step;
  * ``valid`` -- no two records that meet overlap in memory;
  * ``lowest_fit`` -- records placed in a given order, each at the smallest
    aligned offset free of the records already placed that it meets
    (candidate offsets: 0 and the end of every such record);
  * ``greedy_by_size`` -- ``lowest_fit`` in the order (size descending,
    index ascending);
  * ``optimum`` -- the smallest arena over every placement order (brute
    force, n <= 7): a placement sorted by offset and replayed with
    ``lowest_fit`` in that order never grows, so some order reaches the
    optimum;
  * ``lower_bound`` -- the largest sum of rounded sizes alive at one step.
"""
import itertools


def rounded(nbytes, align):
    return -(-int(nbytes) // align) * align


def meets(a_first, a_last, b_first, b_last):
    return a_first <= b_last and b_first <= a_last


def valid(nbytes, first, last, offsets, align=1):
    n = len(nbytes)
    for i in range(n):
        if offsets[i] % align:
            return False
        for j in range(i + 1, n):
            if not meets(first[i], last[i], first[j], last[j]):
                continue
            a0, a1 = offsets[i], offsets[i] + rounded(nbytes[i], align)
            b0, b1 = offsets[j], offsets[j] + rounded(nbytes[j], align)
            if a0 < a1 and b0 < b1 and a0 < b1 and b0 < a1:
                return False
    return True


def arena_size(nbytes, offsets, align=1):
    return max([offsets[i] + rounded(nbytes[i], align) for i in range(len(nbytes))
                if rounded(nbytes[i], align) > 0], default=0)


def lowest_fit(nbytes, first, last, order, align=1):
    offsets = [0] * len(nbytes)
    placed = []
    for i in order:
        size = rounded(nbytes[i], align)
        if size == 0:
            continue
        others = [j for j in placed if meets(first[i], last[i], first[j], last[j])]
        candidates = sorted({0} | {offsets[j] + rounded(nbytes[j], align) for j in others})
        for c in candidates:
            if all(c + size <= offsets[j] or offsets[j] + rounded(nbytes[j], align) <= c
                   for j in others):
                offsets[i] = c
                break
        placed.append(i)
    return offsets


def greedy_by_size(nbytes, first, last, align=1):
    order = sorted(range(len(nbytes)), key=lambda i: (-int(nbytes[i]), i))
    offsets = lowest_fit(nbytes, first, last, order, align)
    return offsets, arena_size(nbytes, offsets, align)


def optimum(nbytes, first, last, align=1):
    n = len(nbytes)
    if n > 7:
        raise ValueError("brute force is for n <= 7")
    best = None
    for order in itertools.permutations(range(n)):
        size = arena_size(nbytes, lowest_fit(nbytes, first, last, order, align), align)
        best = size if best is None else min(best, size)
    return best if best is not None else 0


def lower_bound(nbytes, first, last, align=1):
    steps = sorted(set(first) | set(last))
    return max([sum(rounded(nbytes[i], align) for i in range(len(nbytes)) if first[i] <= s <= last[i])
                for s in steps], default=0)
