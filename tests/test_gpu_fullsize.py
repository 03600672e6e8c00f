"""Parity at the workloads' full sizes, in the launch configuration bench.py times.

Each test scores a workload's whole request stream through es_score_requests
(DP planner at the workload's token budget and batch overhead; bench.py's
default planned batches per pass and passes in flight), then
  * compares EVERY reward with the float64 oracle's reward for that request,
    computed one sequence at a time by tests/golden/make_stream_rewards.py
    (oracle/ and synth/ only) and stored in tests/golden/stream_rewards_*.npy:
    max |error| <= 1e-2 for bf16 models (bf16 operands, fp32 accumulation)
    and <= 1e-5 for the fp32 model; the max, 99th percentile and mean errors
    are printed;
  * checks properties that hold at any size: the stream is bitwise
    reproducible, and a few requests scored alone as one packed batch give
    bitwise the rewards they got inside the stream.
The best-of-16 test checks the per-prompt choice of es_score_best_of_n
against the oracle's rewards: the chosen candidate's oracle reward is within
2e-2 (twice the reward tolerance) of the prompt's oracle maximum, and where
the oracle's best candidate leads the runner-up by more than 2e-2 the choice
is exactly the oracle's.
"""
import functools
import os

import numpy as np
import pytest

import oracle
from bench import launch_config
from encoder_scoring_amd import Scorer, blob
from helpers import need_gpu, offsets_of, say
from synth import get_config, make_fixed_batch, make_requests, make_weights
from synth.generate import best_of_n_form, split

pytestmark = pytest.mark.gpu
BF16_TOL = 1e-2
FP32_TOL = 1e-5
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def golden(name):
    path = os.path.join(GOLDEN, f"stream_rewards_{name}.npy")
    if not os.path.exists(path):
        pytest.fail(f"missing {path}: run python tests/golden/make_stream_rewards.py {name}")
    return np.load(path)


@functools.lru_cache(maxsize=2)
def weights_of(name):
    say(name, ": drawing weights")
    return make_weights(get_config(name))


def _stream(torch, cfg, w, ids, lengths, attention):
    sc = Scorer(blob.to_bytes(cfg, w, 0.0), cfg.max_tokens, min(cfg.max_tokens, 65536))
    group, in_flight = launch_config(cfg.name)
    sc.set_grouping(group)
    sc.set_concurrency(in_flight)
    if cfg.bf16:
        sc.set_attention(attention)
    d = torch.from_numpy(ids).cuda()
    rew, stats = sc.score_requests(d, lengths, cfg.batch_overhead)
    again, _ = sc.score_requests(d, lengths, cfg.batch_overhead)
    torch.cuda.synchronize()
    assert torch.equal(rew, again), "stream not bitwise reproducible"
    r = rew.cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(r))
    say(cfg.name, attention, "stream:", lengths.size, "requests", int(lengths.sum()), "tokens",
        stats["n_batches"], "batches")
    return sc, r


def _compare_all(name, attention, got, want, tol):
    assert got.shape == want.shape
    err = np.abs(got - want)
    worst = int(np.argmax(err))
    say(f"{name} [{attention}]: {err.size} rewards vs oracle: max {err.max():.3e} "
        f"(request {worst}), p99 {np.percentile(err, 99):.3e}, mean {err.mean():.3e}")
    assert err.max() <= tol, f"{name} [{attention}]: request {worst} off by {err.max():.3e}"


def _alone_bitwise(torch, sc, ids, lengths, rew, idx):
    seqs = split(ids, lengths)
    sub = [seqs[i] for i in idx]
    alone = sc.score(torch.from_numpy(np.concatenate(sub)).cuda(), offsets_of([len(s) for s in sub]))
    torch.cuda.synchronize()
    assert np.array_equal(alone.cpu().numpy().astype(np.float64), rew[idx])


def test_tiny_fp32_full_stream():
    torch = need_gpu()
    cfg = get_config("tiny_fp32")
    ids, lengths, _ = make_requests(cfg)
    sc, rew = _stream(torch, cfg, make_weights(cfg), ids, lengths, "unfused")
    _compare_all(cfg.name, "unfused", rew, golden("tiny_fp32"), FP32_TOL)


@pytest.mark.parametrize("attention", ["unfused", "fused"])
@pytest.mark.parametrize("n", [64, 128, 256])
def test_tinybert_fixed_length_batch64(n, attention):
    torch = need_gpu()
    cfg = get_config("tinybert")
    ids, lengths = make_fixed_batch(cfg, n, 64)
    sc, rew = _stream(torch, cfg, weights_of("tinybert"), ids, lengths, attention)
    _compare_all(f"tinybert_b64_n{n}", attention, rew, golden(f"tinybert_b64_n{n}"), BF16_TOL)
    _alone_bitwise(torch, sc, ids, lengths, rew, np.array([0, 31, 63]))


@pytest.mark.parametrize("attention", ["unfused", "fused"])
def test_bert_base_short_full_stream(attention):
    torch = need_gpu()
    cfg = get_config("bert_base_short")
    ids, lengths, _ = make_requests(cfg)
    sc, rew = _stream(torch, cfg, weights_of(cfg.name), ids, lengths, attention)
    _compare_all(cfg.name, attention, rew, golden(cfg.name), BF16_TOL)
    idx = np.random.default_rng(1).choice(lengths.size, 8, replace=False)
    _alone_bitwise(torch, sc, ids, lengths, rew,
                   np.concatenate([idx, [int(np.argmax(lengths)), int(np.argmin(lengths))]]))


@pytest.mark.parametrize("attention", ["unfused", "fused"])
def test_bert_base_longtail_full_stream(attention):
    torch = need_gpu()
    cfg = get_config("bert_base_longtail")
    ids, lengths, _ = make_requests(cfg)
    sc, rew = _stream(torch, cfg, weights_of(cfg.name), ids, lengths, attention)
    _compare_all(cfg.name, attention, rew, golden(cfg.name), BF16_TOL)
    idx = np.random.default_rng(2).choice(lengths.size, 3, replace=False)
    _alone_bitwise(torch, sc, ids, lengths, rew,
                   np.concatenate([idx, [int(np.argmax(lengths)), int(np.argmin(lengths))]]))


@pytest.mark.parametrize("attention", ["unfused", "fused"])
def test_decoder_rm_best_of_16_full_stream(attention):
    torch = need_gpu()
    cfg = get_config("decoder_rm")
    ids, lengths, group = make_requests(cfg)
    sc, rew = _stream(torch, cfg, weights_of(cfg.name), ids, lengths, attention)
    _compare_all(cfg.name, attention, rew, golden(cfg.name), BF16_TOL)
    _alone_bitwise(torch, sc, ids, lengths, rew,
                   np.array([int(np.argmin(lengths)), int(np.argmax(lengths))]))


def test_decoder_rm_reference_offset():
    """Calibration on the reference set (64 prompts + one reference summary
    each): the calibrated offset makes the reference rewards average zero, and
    every stream reward moves by exactly that one fp32 addition."""
    torch = need_gpu()
    from synth import make_reference_set
    cfg = get_config("decoder_rm")
    ids, lengths, _ = make_requests(cfg)
    sc, rew = _stream(torch, cfg, weights_of(cfg.name), ids, lengths, "fused")
    rid, rlen = make_reference_set(cfg)
    d_ref = torch.from_numpy(rid).cuda()
    off = sc.calibrate_offset(d_ref, offsets_of(rlen))
    sc.reward_offset = off
    ref, _ = sc.score_requests(d_ref, rlen, cfg.batch_overhead)
    torch.cuda.synchronize()
    assert abs(float(ref.double().mean())) < 1e-5
    shifted, _ = sc.score_requests(torch.from_numpy(ids).cuda(), lengths, cfg.batch_overhead)
    torch.cuda.synchronize()
    want = (rew.astype(np.float32) + np.float32(off)).astype(np.float64)
    assert np.array_equal(shifted.cpu().numpy().astype(np.float64), want)


def test_decoder_rm_best_of_16_shared_prompts():
    """The decoder workload through es_score_best_of_n (each 512-token prompt
    run once for its 16 candidates): every reward within 1e-2 of the oracle's
    for that prompt + candidate sequence, bitwise equal to scoring the
    concatenated sequences on the GPU, and each prompt's choice valid against
    the oracle's rewards (see the module docstring)."""
    torch = need_gpu()
    cfg = get_config("decoder_rm")
    ids, lengths, group = make_requests(cfg)
    want = golden(cfg.name)
    sc, rew = _stream(torch, cfg, weights_of(cfg.name), ids, lengths, "fused")
    p_ids, pl, c_ids, cl, cn = best_of_n_form(ids, lengths, group, 512)
    d = torch.from_numpy(np.concatenate([p_ids, c_ids])).cuda()
    got, best, stats = sc.score_best_of_n(d, pl, cl, cn, cfg.batch_overhead)
    torch.cuda.synchronize()
    say("shared prompts:", stats)
    got = got.cpu().numpy().astype(np.float64)
    assert np.array_equal(got, rew)
    _compare_all(cfg.name, "shared prompts", got, want, BF16_TOL)
    best = best.cpu().numpy()
    assert best.tolist() == oracle.best_of_n(got.tolist(), cn.tolist())
    starts = np.concatenate([[0], np.cumsum(cn)])
    exact = 0
    for p in range(cn.size):
        o = want[starts[p]:starts[p + 1]]
        top = np.sort(o)[::-1]
        chosen = int(best[p])
        assert 0 <= chosen < cn[p]
        assert o[chosen] >= top[0] - 2 * BF16_TOL, f"prompt {p}: chose {chosen}"
        if top[0] - top[1] > 2 * BF16_TOL:
            assert chosen == int(oracle.best_of_n(o.tolist(), [int(cn[p])])[0]), f"prompt {p}"
            exact += 1
    say(f"best-of-16: {cn.size} prompts valid, {exact} with a clear oracle winner matched exactly")
    assert stats["packed_tokens"] == int(pl.sum() + cl.sum())
