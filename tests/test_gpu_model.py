"""End-to-end parity of the HIP scoring path against the oracle (small inputs).

Bars: rewards max-abs <= 1e-5 for fp32 models and <= 1e-2 for bf16 models
(bf16 GEMM operands, fp32 accumulation); plans and offsets bit-exact; the GPU
result for a sequence does not depend on the rest of its batch (bitwise).
"""
import numpy as np
import pytest

import oracle
from encoder_scoring_amd import EncScoreError, Scorer, blob
from helpers import mini, need_gpu, offsets_of, say
from synth import get_config, make_fixed_batch, make_reference_set, make_requests, make_weights
from synth.generate import random_stream, split

pytestmark = pytest.mark.gpu

FP32_TOL = 1e-5
BF16_TOL = 1e-2


def scorer_for(cfg, w, offset=0.0, max_tokens=4096, max_seqs=512):
    return Scorer(blob.to_bytes(cfg, w, offset), max_tokens, max_seqs)


def gpu_score(torch, sc, ids, lengths):
    d = torch.from_numpy(np.ascontiguousarray(ids, dtype=np.int32)).cuda()
    r = sc.score(d, offsets_of(lengths))
    torch.cuda.synchronize()
    return r.cpu().numpy().astype(np.float64)


CASES = [
    ("tiny_fp32", get_config("tiny_fp32"), FP32_TOL),
    ("dec_fp32", mini("dec_fp32", True, True, False, H=128, A=2, F=256, P=128), FP32_TOL),
    ("enc_fp32_d26", mini("enc_fp32_d26", False, False, False, H=52, A=2, F=96, P=80), FP32_TOL),
    ("dec_bf16_d128", mini("dec_bf16_d128", True, True, True, H=256, A=2, F=512, V=1000, P=300), BF16_TOL),
    ("enc_bf16", mini("enc_bf16", False, False, True, H=192, A=3, F=384, V=500, P=200), BF16_TOL),
]


ATTENTION_CASES = [(n, c, t, a) for n, c, t in CASES for a in (["unfused", "fused"] if c.bf16 else ["unfused"])]


@pytest.mark.parametrize("name,cfg,tol,attention", ATTENTION_CASES,
                         ids=[f"{c[0]}-{c[3]}" for c in ATTENTION_CASES])
def test_rewards_match_oracle(name, cfg, tol, attention):
    torch = need_gpu()
    say("rewards", name, attention)
    w = make_weights(cfg)
    ids, lengths = random_stream(5, 11, 1, min(cfg.max_pos, 150), cfg.vocab)
    sc = scorer_for(cfg, w, offset=0.125)
    sc.set_attention(attention)
    got = gpu_score(torch, sc, ids, lengths)
    want = oracle.OracleModel(cfg, w).score_many(split(ids, lengths), 0.125)
    say(name, "max |d reward| =", float(np.max(np.abs(got - want))))
    assert np.max(np.abs(got - want)) <= tol


@pytest.mark.parametrize("name,cfg,tol", CASES[:3], ids=[c[0] for c in CASES[:3]])
def test_hidden_states_match_oracle_fp32(name, cfg, tol):
    torch = need_gpu()
    w = make_weights(cfg)
    ids, lengths = random_stream(6, 5, 1, min(cfg.max_pos, 90), cfg.vocab)
    sc = scorer_for(cfg, w)
    m = oracle.OracleModel(cfg, w)
    d = torch.from_numpy(ids).cuda()
    for L in range(cfg.n_layers + 1):
        got = sc.hidden(d, offsets_of(lengths), L).cpu().numpy()
        want = np.concatenate([m.hidden(s, L) for s in split(ids, lengths)])
        err = np.max(np.abs(got - want))
        say(name, "layer", L, "max |d hidden| =", float(err))
        assert err < 2e-5 * max(1.0, float(np.max(np.abs(want))))


def test_tiny_workload_and_calibration():
    torch = need_gpu()
    cfg = get_config("tiny_fp32")
    w = make_weights(cfg)
    m = oracle.OracleModel(cfg, w)
    rid, rlen = make_reference_set(cfg)
    off_oracle = m.calibrate_offset(split(rid, rlen))
    sc = scorer_for(cfg, w, 0.0, max_tokens=1024, max_seqs=64)
    off_gpu = sc.calibrate_offset(torch.from_numpy(rid).cuda(), offsets_of(rlen))
    assert abs(off_gpu - off_oracle) <= FP32_TOL
    sc.reward_offset = off_gpu
    ref = gpu_score(torch, sc, rid, rlen)
    assert abs(ref.mean()) < 1e-6
    ids, lengths, _ = make_requests(cfg)
    got = gpu_score(torch, sc, ids, lengths)
    want = m.score_many(split(ids, lengths), off_gpu)
    assert np.max(np.abs(got - want)) <= FP32_TOL


def test_tinybert_fixed_lengths():
    torch = need_gpu()
    cfg = get_config("tinybert")
    w = make_weights(cfg)
    m = oracle.OracleModel(cfg, w)
    sc = scorer_for(cfg, w, 0.0, max_tokens=16384, max_seqs=64)
    for n, B in [(64, 1), (128, 1), (256, 1), (64, 8), (256, 3)]:
        ids, lengths = make_fixed_batch(cfg, n, B)
        got = gpu_score(torch, sc, ids, lengths)
        want = m.score_many(split(ids, lengths))
        say("tinybert", n, B, float(np.max(np.abs(got - want))))
        assert np.max(np.abs(got - want)) <= BF16_TOL


def test_bert_base_short_sample():
    torch = need_gpu()
    cfg = get_config("bert_base_short")
    w = make_weights(cfg)
    ids, lengths, _ = make_requests(cfg)
    seqs = split(ids, lengths)[:6]
    sc = scorer_for(cfg, w, 0.0, max_tokens=4096, max_seqs=2048)
    got = gpu_score(torch, sc, np.concatenate(seqs), [len(s) for s in seqs])
    want = oracle.OracleModel(cfg, w).score_many(seqs)
    say("bert_base sample", float(np.max(np.abs(got - want))))
    assert np.max(np.abs(got - want)) <= BF16_TOL


@pytest.mark.parametrize("cfg,attention", [(CASES[0][1], "unfused"), (CASES[3][1], "unfused"),
                                           (CASES[3][1], "fused"), (CASES[4][1], "fused")],
                         ids=["fp32", "bf16_causal-unfused", "bf16_causal-fused", "bf16_enc-fused"])
def test_batch_invariance_and_determinism(cfg, attention):
    torch = need_gpu()
    w = make_weights(cfg)
    ids, lengths = random_stream(8, 9, 1, min(cfg.max_pos, 120), cfg.vocab)
    sc = scorer_for(cfg, w)
    sc.set_attention(attention)
    packed = gpu_score(torch, sc, ids, lengths)
    again = gpu_score(torch, sc, ids, lengths)
    assert np.array_equal(packed, again)                       # run to run, bitwise
    alone = np.array([gpu_score(torch, sc, s, [len(s)])[0] for s in split(ids, lengths)])
    assert np.array_equal(packed, alone)                       # batch composition, bitwise
    perm = np.random.default_rng(0).permutation(len(lengths))
    seqs = split(ids, lengths)
    pids = np.concatenate([seqs[i] for i in perm])
    assert np.array_equal(gpu_score(torch, sc, pids, lengths[perm]), packed[perm])


def test_score_requests_matches_batches_and_oracle():
    torch = need_gpu()
    cfg = CASES[4][1]
    w = make_weights(cfg)
    ids, lengths = random_stream(9, 40, 1, 120, cfg.vocab)
    T = 512
    sc = scorer_for(cfg, w, 0.5, max_tokens=T, max_seqs=512)
    d = torch.from_numpy(ids).cuda()
    rew, stats = sc.score_requests(d, lengths, batch_overhead=64)
    torch.cuda.synchronize()
    rew = rew.cpu().numpy().astype(np.float64)
    order, starts, cost = oracle.plan_batches(lengths, T, 64)
    assert stats["n_batches"] == len(starts) - 1 and stats["total_cost"] == cost
    assert stats["packed_tokens"] == int(lengths.sum())
    seqs = split(ids, lengths)
    for b in range(len(starts) - 1):
        idx = order[starts[b]:starts[b + 1]]
        sub = gpu_score(torch, sc, np.concatenate([seqs[i] for i in idx]), lengths[idx])
        assert np.array_equal(sub, rew[idx])
    want = oracle.OracleModel(cfg, w).score_many(seqs, 0.5)
    assert np.max(np.abs(rew - want)) <= BF16_TOL


def test_host_validation_errors():
    torch = need_gpu()
    cfg = CASES[0][1]
    sc = scorer_for(cfg, make_weights(cfg), max_tokens=100, max_seqs=4)
    d = torch.zeros(200, dtype=torch.int32, device="cuda")
    bad = [
        (np.array([1, 3]), -1),          # offsets[0] != 0
        (np.array([0, 3, 3]), -1),       # empty sequence
        (np.array([0, 65]), -2),         # longer than max_pos (64)
        (np.array([0, 60, 120]), -3),    # above max_tokens
        (np.array([0, 1, 2, 3, 4, 5]), -3),  # above max_seqs
    ]
    for off, code in bad:
        with pytest.raises(EncScoreError) as e:
            sc.score(d, off)
        assert e.value.status == code, (off, str(e.value))
    ok = sc.score(d[:10], np.array([0, 4, 10]))
    torch.cuda.synchronize()
    assert np.all(np.isfinite(ok.cpu().numpy()))


def test_out_of_range_token_sets_device_flag():
    torch = need_gpu()
    cfg = CASES[0][1]
    sc = scorer_for(cfg, make_weights(cfg), max_tokens=100, max_seqs=4)
    sc.check_device_errors()
    d = torch.tensor([1, 2, cfg.vocab + 5, 3], dtype=torch.int32, device="cuda")
    r = sc.score(d, np.array([0, 4]))
    with pytest.raises(EncScoreError) as e:
        sc.check_device_errors()
    assert e.value.status == -7
    sc.check_device_errors()                     # flag was cleared
    assert np.isfinite(r.cpu().numpy()).all()


@pytest.mark.parametrize("lanes", [2, 3])
def test_batches_in_flight_match_serial(lanes):
    """Overlapping planned batches on internal streams changes nothing (bitwise).
    The model is a pre-LN bf16 decoder, so this also pins the last-token
    refinement on its own stream (one pass in flight) against the refinement
    on the pass's stream (several in flight)."""
    torch = need_gpu()
    cfg = CASES[3][1]
    w = make_weights(cfg)
    ids, lengths = random_stream(10, 60, 1, 200, cfg.vocab)
    sc = scorer_for(cfg, w, 0.25, max_tokens=600, max_seqs=512)
    d = torch.from_numpy(ids).cuda()
    serial, st1 = sc.score_requests(d, lengths, batch_overhead=64)
    serial = serial.clone()
    sc.set_concurrency(lanes)
    for _ in range(2):
        par, st2 = sc.score_requests(d, lengths, batch_overhead=64)
        torch.cuda.synchronize()
        assert st2 == st1 and st1["n_batches"] > lanes
        assert torch.equal(par, serial)
    sc.set_concurrency(1)
    again, _ = sc.score_requests(d, lengths, batch_overhead=64)
    assert torch.equal(again, serial)


@pytest.mark.parametrize("name,cfg,tol", CASES, ids=[c[0] for c in CASES])
@pytest.mark.parametrize("attention", ["unfused", "fused"])
def test_last_layer_pruning_is_bitwise_exact(name, cfg, tol, attention):
    """The last layer on the last tokens only gives bitwise the rewards of the
    full last layer (es_score_batch and es_score_requests), for every model
    form and both attention forms."""
    torch = need_gpu()
    if attention == "fused" and not cfg.bf16:
        pytest.skip("fused attention needs a bf16 model")
    w = make_weights(cfg)
    ids, lengths = random_stream(17, 23, 1, min(cfg.max_pos, 120), cfg.vocab)
    sc = scorer_for(cfg, w, offset=0.5, max_tokens=3000)
    if cfg.bf16:
        sc.set_attention(attention)
    d = torch.from_numpy(ids).cuda()
    sc.set_pruning(False)
    full_b = gpu_score(torch, sc, ids, lengths)
    full_s, st = sc.score_requests(d, lengths, batch_overhead=32)
    full_s = full_s.clone()
    sc.set_pruning(True)
    assert np.array_equal(gpu_score(torch, sc, ids, lengths), full_b)
    pr_s, _ = sc.score_requests(d, lengths, batch_overhead=32)
    torch.cuda.synchronize()
    say(name, attention, "pruned vs full:", st["n_batches"], "batches")
    assert torch.equal(pr_s, full_s)


@pytest.mark.parametrize("group,lanes", [(2, 1), (3, 1), (4, 2), (8, 1)])
@pytest.mark.parametrize("attention", ["unfused", "fused"])
def test_batch_grouping_matches_ungrouped(group, lanes, attention):
    """Packing G planned batches into one pass changes nothing (bitwise), with
    and without passes in flight, for both attention forms."""
    torch = need_gpu()
    cfg = CASES[3][1]
    w = make_weights(cfg)
    ids, lengths = random_stream(11, 70, 1, 200, cfg.vocab)
    sc = scorer_for(cfg, w, 0.25, max_tokens=600, max_seqs=512)
    sc.set_attention(attention)
    d = torch.from_numpy(ids).cuda()
    ref, st1 = sc.score_requests(d, lengths, batch_overhead=64)
    ref = ref.clone()
    say("grouping", group, "lanes", lanes, attention, st1["n_batches"], "planned batches")
    assert st1["n_batches"] > group
    sc.set_grouping(group)
    sc.set_concurrency(lanes)
    for _ in range(2):
        got, st2 = sc.score_requests(d, lengths, batch_overhead=64)
        torch.cuda.synchronize()
        assert st2 == st1
        assert torch.equal(got, ref)
    sc.set_grouping(1)
    sc.set_concurrency(1)
    again, _ = sc.score_requests(d, lengths, batch_overhead=64)
    assert torch.equal(again, ref)


def test_grouping_and_concurrency_validation():
    torch = need_gpu()
    from encoder_scoring_amd import EncScoreError
    cfg = CASES[0][1]
    sc = scorer_for(cfg, make_weights(cfg), 0.0)
    for bad in (0, 9, -1):
        with pytest.raises(EncScoreError):
            sc.set_grouping(bad)
    for bad in (0, 5):
        with pytest.raises(EncScoreError):
            sc.set_concurrency(bad)
    from encoder_scoring_amd._lib import check
    with pytest.raises(EncScoreError):
        check(sc.lib, sc.lib.es_set_pruning(sc.handle, 2))


@pytest.mark.parametrize("name,cfg", [(c[0], c[1]) for c in CASES if c[1].bf16],
                         ids=[c[0] for c in CASES if c[1].bf16])
def test_fused_attention_matches_oracle_and_unfused(name, cfg):
    """The fused attention kernel: same rewards as the oracle (1e-2) and close
    to the three-kernel path (both round P to bf16, in different places)."""
    torch = need_gpu()
    w = make_weights(cfg)
    ids, lengths = random_stream(15, 13, 1, min(cfg.max_pos, 200), cfg.vocab)
    sc = scorer_for(cfg, w, offset=0.125)
    fused_default = gpu_score(torch, sc, ids, lengths)     # bf16 models default to fused
    sc.set_attention("unfused")
    unfused = gpu_score(torch, sc, ids, lengths)
    sc.set_attention("fused")
    fused = gpu_score(torch, sc, ids, lengths)
    assert np.array_equal(fused, gpu_score(torch, sc, ids, lengths))
    assert np.array_equal(fused, fused_default)
    want = oracle.OracleModel(cfg, w).score_many(split(ids, lengths), 0.125)
    say(name, "fused max |d| =", float(np.max(np.abs(fused - want))),
        "vs unfused", float(np.max(np.abs(fused - unfused))))
    assert np.max(np.abs(fused - want)) <= BF16_TOL
    assert np.max(np.abs(fused - unfused)) <= 5e-3
    sc.set_attention("unfused")
    assert np.array_equal(gpu_score(torch, sc, ids, lengths), unfused)


def test_fused_attention_hidden_states():
    torch = need_gpu()
    cfg = CASES[3][1]          # causal pre-LN, head dim 128
    w = make_weights(cfg)
    ids, lengths = random_stream(16, 7, 1, 150, cfg.vocab)
    sc = scorer_for(cfg, w)
    sc.set_attention("fused")
    m = oracle.OracleModel(cfg, w)
    got = sc.hidden(torch.from_numpy(ids).cuda(), offsets_of(lengths), 1).cpu().numpy()
    want = np.concatenate([m.hidden(s, 1) for s in split(ids, lengths)])
    assert np.max(np.abs(got - want)) < 0.05 * max(1.0, float(np.max(np.abs(want))))


def test_refinement_switch_and_effect():
    """The last-token refinement: on by default for a pre-LN bf16 model and
    refused for a post-LN one; with it the rewards sit closer to the float64
    oracle (the reward rows carry no bf16 operand rounding) than the bf16
    pass's own (es_set_refinement(0)), both within the bf16 bar, and pruning
    gives the same bits either way."""
    torch = need_gpu()
    cfg = mini("dec_bf16_deep", True, True, True, H=256, A=2, F=1024, L=8, V=1000, P=300)
    w = make_weights(cfg)
    ids, lengths = random_stream(21, 24, 20, 250, cfg.vocab)
    sc = scorer_for(cfg, w)
    assert sc.refinement()
    want = oracle.OracleModel(cfg, w).score_many(split(ids, lengths), 0.0)
    errs = {}
    for on in (True, False):
        sc.set_refinement(on)
        assert sc.refinement() == on
        got = gpu_score(torch, sc, ids, lengths)
        sc.set_pruning(False)
        assert np.array_equal(gpu_score(torch, sc, ids, lengths), got)
        sc.set_pruning(True)
        errs[on] = np.abs(got - want)
        say("refinement", on, "max", float(errs[on].max()), "mean", float(errs[on].mean()))
        assert errs[on].max() <= BF16_TOL
    assert errs[True].max() < errs[False].max() and errs[True].mean() < errs[False].mean()
    enc = CASES[4][1]
    sc2 = scorer_for(enc, make_weights(enc))
    assert not sc2.refinement()
    sc2.set_refinement(False)
    with pytest.raises(EncScoreError):
        sc2.set_refinement(True)


@pytest.mark.parametrize("attention", ["unfused", "fused"])
def test_refinement_at_the_longest_sequences(attention):
    """A pre-LN bf16 model at max_pos = 1024 (the weight format's limit, which
    the last-token attention holds): a 1024-token sequence next to 1-token and mid-length
    ones, rewards against the oracle within the bf16 bar, and bitwise the same
    when each sequence is scored alone."""
    torch = need_gpu()
    cfg = mini("dec_long", True, True, True, H=128, A=2, F=256, V=500, P=1024)
    w = make_weights(cfg)
    lengths = np.array([1024, 1, 333, 700, 2], dtype=np.int32)
    rng = np.random.default_rng(44)
    ids = rng.integers(0, cfg.vocab, size=int(lengths.sum())).astype(np.int32)
    sc = scorer_for(cfg, w, max_tokens=4096, max_seqs=16)
    assert sc.refinement()
    sc.set_attention(attention)
    got = gpu_score(torch, sc, ids, lengths)
    want = oracle.OracleModel(cfg, w).score_many(split(ids, lengths), 0.0)
    say("dec_long", attention, "max |d reward| =", float(np.max(np.abs(got - want))))
    assert np.max(np.abs(got - want)) <= BF16_TOL
    for i, s in enumerate(split(ids, lengths)):
        assert gpu_score(torch, sc, s, np.array([s.size], dtype=np.int32))[0] == got[i]
