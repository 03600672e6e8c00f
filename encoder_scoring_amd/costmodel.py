"""Measured batch-cost table for the DP batch planner.

TurboTransformers review (Abstract; Proposed method): the batch scheduler
groups variable-length requests by dynamic programming for throughput.  Its
cost of a batch here is what a batch of that shape was measured to take on
the GPU: ``measure_cost_grid`` times one forward pass (``Scorer.score``, one
packed batch) of b sequences of l tokens on a coarse (b, l) grid, and
``dense_cost_table`` turns the grid into the dense table
``es_plan_batches_measured`` / ``Scorer.set_cost_table`` take:
table[b-1, l-1] in integer nanoseconds.

Host logic only (interpolation and integer rounding); the timed work is the
library's own forward pass.
"""
import numpy as np


def _interp_extrap(x, xp, fp):
    """Piecewise-linear interpolation of (xp, fp) at x, extended linearly
    beyond both ends (a single point is taken as proportional to x)."""
    xp = np.asarray(xp, dtype=np.float64)
    fp = np.asarray(fp, dtype=np.float64)
    x = np.asarray(x, dtype=np.float64)
    if xp.size == 1:
        return fp[0] * x / xp[0]
    y = np.interp(x, xp, fp)
    lo, hi = x < xp[0], x > xp[-1]
    y[lo] = fp[0] + (x[lo] - xp[0]) * (fp[1] - fp[0]) / (xp[1] - xp[0])
    y[hi] = fp[-1] + (x[hi] - xp[-1]) * (fp[-1] - fp[-2]) / (xp[-1] - xp[-2])
    return y


def dense_cost_table(batch_grid, len_grid, measured_ms, max_len):
    """Dense int64 table [max(batch_grid), max_len] in nanoseconds.

    measured_ms[i, j] is the time of batch_grid[i] sequences of len_grid[j]
    tokens (NaN where not measured, e.g. beyond the token budget).  Each
    measured length column is interpolated piecewise-linearly in the batch
    size (extended linearly past its last measured size), then every batch
    size is interpolated the same way along the length.  Entries are clipped
    at zero and made non-decreasing along the length (a running maximum),
    which the planner requires.
    """
    bg = np.asarray(batch_grid, dtype=np.int64)
    lg = np.asarray(len_grid, dtype=np.int64)
    meas = np.asarray(measured_ms, dtype=np.float64)
    if meas.shape != (bg.size, lg.size):
        raise ValueError(f"measured_ms has shape {meas.shape}, want {(bg.size, lg.size)}")
    if np.any(np.diff(bg) <= 0) or np.any(np.diff(lg) <= 0) or bg[0] < 1 or lg[0] < 1:
        raise ValueError("grids must be strictly increasing and start at >= 1")
    max_batch = int(bg[-1])
    sizes = np.arange(1, max_batch + 1)
    cols = []
    used = []
    for j in range(lg.size):
        ok = ~np.isnan(meas[:, j])
        if not ok.any():
            continue
        cols.append(_interp_extrap(sizes, bg[ok], meas[ok, j]))
        used.append(int(lg[j]))
    if not cols:
        raise ValueError("no measured point")
    by_len = np.stack(cols, axis=1)                           # [max_batch, len. used]
    lens = np.arange(1, max_len + 1)
    ms = np.empty((max_batch, max_len))
    for b in range(max_batch):
        if len(used) == 1:
            ms[b] = by_len[b, 0]
        else:
            ms[b] = _interp_extrap(lens, used, by_len[b])
        ms[b, lens < used[0]] = by_len[b, 0]                  # shorter than measured: no cheaper
    ns = np.rint(np.clip(ms, 0.0, None) * 1e6).astype(np.int64)
    return np.maximum.accumulate(ns, axis=1)


def measure_cost_grid(scorer, batch_grid, len_grid, reps=5, warmup=2, seed=0):
    """Median time (ms) of one forward pass of b sequences of l tokens (ids
    drawn uniformly from the vocabulary) for every (b, l) of the grids that
    the handle can score in one batch -- b <= max_seqs, l <= max_pos,
    b * l <= max_tokens -- and NaN elsewhere; timed with events on the
    current stream."""
    import torch
    info = scorer.info
    rng = np.random.default_rng(seed)
    out = np.full((len(batch_grid), len(len_grid)), np.nan)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for i, b in enumerate(batch_grid):
        for j, l in enumerate(len_grid):
            if b > info.max_seqs or l > info.max_pos or b * l > info.max_tokens:
                continue
            ids = rng.integers(0, info.vocab, size=b * l).astype(np.int32)
            d_ids = torch.from_numpy(ids).cuda()
            offsets = (np.arange(b + 1) * l).astype(np.int32)
            rew = torch.empty(b, dtype=torch.float32, device="cuda")
            times = []
            for r in range(warmup + reps):
                ev0.record()
                scorer.score(d_ids, offsets, out=rew)
                ev1.record()
                ev1.synchronize()
                if r >= warmup:
                    times.append(ev0.elapsed_time(ev1))
            out[i, j] = float(np.median(times))
    return out
