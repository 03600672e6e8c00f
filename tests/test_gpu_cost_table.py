"""Measured-cost planning for es_score_requests (es_set_cost_table) on the GPU.

TurboTransformers review, Proposed method: the DP batch scheduler groups
variable-length requests for throughput; with a cost table the cost of a
batch is what a batch of that shape was measured to take.  Checks, through
the C ABI:
  * rewards are bitwise the same under any plan (every kernel works per token
    or per sequence), and the call's plan statistics are those of the
    oracle's table planner on the same lengths and table (rows capped at the
    handle's max_seqs);
  * a table measured on the GPU (Scorer.score on a coarse grid, then the
    dense table) is valid for the planner and plans the stream;
  * NULL goes back to the linear cost; bad tables are rejected.
"""
import numpy as np
import pytest

import oracle
from encoder_scoring_amd import EncScoreError, Scorer, blob
from encoder_scoring_amd.costmodel import dense_cost_table, measure_cost_grid
from helpers import mini, need_gpu, say
from synth import make_weights
from synth.generate import random_stream

pytestmark = pytest.mark.gpu

CFG = mini("enc_bf16_cost", False, False, True, H=192, A=3, F=384, V=500, P=200)
T, MAX_SEQS = 1500, 48


def run(torch, sc, d, lengths, overhead=64):
    r, st = sc.score_requests(d, lengths, batch_overhead=overhead)
    torch.cuda.synchronize()
    return r.clone(), st


def test_cost_table_plans_and_keeps_rewards():
    torch = need_gpu()
    sc = Scorer(blob.to_bytes(CFG, make_weights(CFG), 0.0), T, MAX_SEQS)
    sc.set_attention("fused")
    sc.set_grouping(2)
    ids, lengths = random_stream(41, 200, 1, 200, CFG.vocab)
    d = torch.from_numpy(ids).cuda()
    base, st0 = run(torch, sc, d, lengths)
    rng = np.random.default_rng(3)
    # a made-up table with a large per-batch cost up to 32 sequences, then a
    # steep one: the plan differs from the linear one
    b = np.arange(1, 65, dtype=np.int64)[:, None]
    l = np.arange(1, CFG.max_pos + 1, dtype=np.int64)[None, :]
    table = 5000 + 3 * b * l + np.where(b > 32, 400 * b * l, 0)
    table = np.maximum.accumulate(table + rng.integers(0, 50, size=table.shape), axis=1)
    sc.set_cost_table(table)
    got, st = run(torch, sc, d, lengths)
    assert torch.equal(got, base)
    _, starts, cost = oracle.plan_batches_table(lengths, T, table[:MAX_SEQS])
    say("linear plan", st0["n_batches"], "batches; table plan", st["n_batches"])
    assert st["n_batches"] == len(starts) - 1 and st["total_cost"] == cost
    assert st["n_batches"] != st0["n_batches"]
    sc.set_cost_table(None)
    again, st2 = run(torch, sc, d, lengths)
    assert torch.equal(again, base) and st2 == st0


def test_measured_table_end_to_end():
    torch = need_gpu()
    sc = Scorer(blob.to_bytes(CFG, make_weights(CFG), 0.0), T, MAX_SEQS)
    bg, lg = [1, 4, 16, 48, 64], [8, 32, 100, 200, 256]      # 64 > max_seqs, 256 > max_pos
    meas = measure_cost_grid(sc, bg, lg, reps=3, warmup=1)
    say("measured grid (ms):", np.round(meas, 3).tolist())
    for i, bb in enumerate(bg):
        for j, ll in enumerate(lg):
            assert np.isnan(meas[i, j]) == (bb * ll > T or bb > MAX_SEQS or ll > CFG.max_pos)
    assert np.all(meas[~np.isnan(meas)] > 0)
    table = dense_cost_table(bg, lg, meas, CFG.max_pos)
    assert table.shape == (64, CFG.max_pos)
    ids, lengths = random_stream(42, 150, 1, 200, CFG.vocab)
    d = torch.from_numpy(ids).cuda()
    base, _ = run(torch, sc, d, lengths)
    sc.set_cost_table(table)
    got, st = run(torch, sc, d, lengths)
    assert torch.equal(got, base)
    _, starts, cost = oracle.plan_batches_table(lengths, T, table[:MAX_SEQS])
    assert st["n_batches"] == len(starts) - 1 and st["total_cost"] == cost


def test_bad_cost_tables_rejected():
    torch = need_gpu()
    sc = Scorer(blob.to_bytes(CFG, make_weights(CFG), 0.0), T, MAX_SEQS)
    with pytest.raises(EncScoreError):
        sc.set_cost_table(np.ones((4, CFG.max_pos - 1), dtype=np.int64))     # shorter than max_pos
    falling = np.ones((4, CFG.max_pos), dtype=np.int64)
    falling[2, 7] = 0
    with pytest.raises(EncScoreError):
        sc.set_cost_table(falling)
    ids, lengths = random_stream(43, 20, 1, 200, CFG.vocab)
    d = torch.from_numpy(ids).cuda()
    _, st = run(torch, sc, d, lengths)                  # still the linear planner
    assert st["total_cost"] == oracle.plan_batches(lengths, T, 64)[2]
