"""Parity at the workloads' full sizes, in the launch configuration bench.py times.

Each test scores a workload's whole request stream through es_score_requests
(DP planner at the workload's token budget and batch overhead; four planned
batches packed per pass and two passes in flight, the bench default), then
  * compares a seeded sample of requests, computed one by one by the float64
    oracle, within 1e-2 (bf16 operands, fp32 accumulation);
  * checks properties that hold at any size: every reward finite, the sampled
    requests scored alone as one packed batch give bitwise the same rewards
    as inside the stream, and the stream is bitwise reproducible.
"""
import numpy as np
import pytest

import oracle
from encoder_scoring_amd import Scorer, blob
from helpers import need_gpu, offsets_of, say
from synth import get_config, make_fixed_batch, make_reference_set, make_requests, make_weights
from synth.generate import split

pytestmark = pytest.mark.gpu
BF16_TOL = 1e-2
IN_FLIGHT = 2
GROUP = 4


def _stream(torch, cfg, w, ids, lengths, offset=0.0, attention="fused"):
    sc = Scorer(blob.to_bytes(cfg, w, offset), cfg.max_tokens, min(cfg.max_tokens, 65536))
    sc.set_grouping(GROUP)
    sc.set_concurrency(IN_FLIGHT)
    sc.set_attention(attention)
    d = torch.from_numpy(ids).cuda()
    rew, stats = sc.score_requests(d, lengths, cfg.batch_overhead)
    again, _ = sc.score_requests(d, lengths, cfg.batch_overhead)
    torch.cuda.synchronize()
    assert torch.equal(rew, again), "stream not bitwise reproducible"
    r = rew.cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(r))
    say(cfg.name, "stream:", lengths.size, "requests", int(lengths.sum()), "tokens",
        stats["n_batches"], "batches")
    return sc, r


def _check_sample(torch, sc, cfg, w, ids, lengths, rew, idx, cache=True):
    seqs = split(ids, lengths)
    sub = [seqs[i] for i in idx]
    alone = sc.score(torch.from_numpy(np.concatenate(sub)).cuda(), offsets_of([len(s) for s in sub]))
    torch.cuda.synchronize()
    assert np.array_equal(alone.cpu().numpy().astype(np.float64), rew[idx])
    m = oracle.OracleModel(cfg, w, cache=cache)
    worst = 0.0
    for i in idx:
        want = m.score(seqs[i])
        err = abs(rew[i] - want)
        say(cfg.name, "request", int(i), "len", int(lengths[i]), "gpu", float(rew[i]),
            "oracle", want, "err", err)
        worst = max(worst, err)
    assert worst <= BF16_TOL


@pytest.mark.parametrize("attention", ["unfused", "fused"])
def test_bert_base_short_full_stream(attention):
    torch = need_gpu()
    cfg = get_config("bert_base_short")
    w = make_weights(cfg)
    ids, lengths, _ = make_requests(cfg)
    sc, rew = _stream(torch, cfg, w, ids, lengths, attention=attention)
    idx = np.random.default_rng(1).choice(lengths.size, 8, replace=False)
    idx = np.concatenate([idx, [int(np.argmax(lengths)), int(np.argmin(lengths))]])
    _check_sample(torch, sc, cfg, w, ids, lengths, rew, idx)


@pytest.mark.parametrize("attention", ["unfused", "fused"])
def test_bert_base_longtail_full_stream(attention):
    torch = need_gpu()
    cfg = get_config("bert_base_longtail")
    w = make_weights(cfg)
    ids, lengths, _ = make_requests(cfg)
    sc, rew = _stream(torch, cfg, w, ids, lengths, attention=attention)
    idx = np.random.default_rng(2).choice(lengths.size, 3, replace=False)
    idx = np.concatenate([idx, [int(np.argmax(lengths)), int(np.argmin(lengths))]])
    _check_sample(torch, sc, cfg, w, ids, lengths, rew, idx)


@pytest.mark.parametrize("n", [64, 128, 256])
def test_tinybert_fixed_length_batch64(n):
    torch = need_gpu()
    cfg = get_config("tinybert")
    w = make_weights(cfg)
    ids, lengths = make_fixed_batch(cfg, n, 64)
    sc, rew = _stream(torch, cfg, w, ids, lengths)
    _check_sample(torch, sc, cfg, w, ids, lengths, rew, np.array([0, 31, 63]))


@pytest.mark.parametrize("attention", ["unfused", "fused"])
def test_decoder_rm_best_of_16_full_stream(attention):
    torch = need_gpu()
    cfg = get_config("decoder_rm")
    say("decoder_rm: drawing 1.4B weights")
    w = make_weights(cfg)
    ids, lengths, group = make_requests(cfg)
    sc, rew = _stream(torch, cfg, w, ids, lengths, attention=attention)
    # calibration on the reference set (64 x ~540 tokens, several batches)
    rid, rlen = make_reference_set(cfg)
    d_ref = torch.from_numpy(rid).cuda()
    off = sc.calibrate_offset(d_ref, offsets_of(rlen))
    sc.reward_offset = off
    ref, _ = sc.score_requests(d_ref, rlen, cfg.batch_overhead)
    torch.cuda.synchronize()
    assert abs(float(ref.double().mean())) < 1e-5
    # rewards shift by exactly the offset (one fp32 addition)
    shifted, _ = sc.score_requests(torch.from_numpy(ids).cuda(), lengths, cfg.batch_overhead)
    torch.cuda.synchronize()
    assert np.allclose(shifted.cpu().numpy().astype(np.float64), rew + off, atol=1e-6)
    sc.reward_offset = 0.0
    idx = np.array([int(np.argmin(lengths)), int(np.argmax(lengths))])
    _check_sample(torch, sc, cfg, w, ids, lengths, rew, idx, cache=False)


def test_decoder_rm_best_of_16_shared_prompts():
    """The decoder workload through es_score_best_of_n (each 512-token prompt
    run once for its 16 candidates): rewards bitwise equal to scoring the
    prompt + candidate sequences (fused attention, same launch settings; those
    are oracle-checked in the stream test above), and the per-prompt choice
    equals the oracle's selection on them."""
    torch = need_gpu()
    from synth.generate import best_of_n_form
    cfg = get_config("decoder_rm")
    say("decoder_rm: drawing 1.4B weights")
    w = make_weights(cfg)
    ids, lengths, group = make_requests(cfg)
    sc, rew = _stream(torch, cfg, w, ids, lengths, attention="fused")
    p_ids, pl, c_ids, cl, cn = best_of_n_form(ids, lengths, group, 512)
    d = torch.from_numpy(np.concatenate([p_ids, c_ids])).cuda()
    got, best, stats = sc.score_best_of_n(d, pl, cl, cn, cfg.batch_overhead)
    torch.cuda.synchronize()
    say("shared prompts:", stats)
    assert np.array_equal(got.cpu().numpy().astype(np.float64), rew)
    assert best.cpu().numpy().tolist() == oracle.best_of_n(rew.tolist(), cn.tolist())
    assert stats["packed_tokens"] == int(pl.sum() + cl.sum())
