"""Best-of-N scoring with shared prompts (es_score_best_of_n) on the GPU.

"Learning to summarize from human feedback", Method adaptation: the reward
model scores N candidate summaries of a post and the highest-scoring one is
kept.  Checks, through the C ABI:
  * every candidate's reward equals, bitwise, the reward es_score_requests
    gives for the prompt + candidate laid out as one sequence (fused
    attention), with and without grouping / passes in flight;
  * rewards within 1e-2 of the float64 oracle on prompt + candidate;
  * the chosen index per prompt equals the oracle's selection on those
    rewards (ties -> lowest index), including exact ties;
  * host validation errors.
"""
import numpy as np
import pytest

import oracle
from encoder_scoring_amd import EncScoreError, Scorer, blob
from helpers import mini, need_gpu, say
from synth import make_weights

pytestmark = pytest.mark.gpu
BF16_TOL = 1e-2

DEC64 = mini("dec_bf16_d64", True, True, True, H=256, A=4, F=512, V=1000, P=300, seed=21)
DEC128 = mini("dec_bf16_d128", True, True, True, H=256, A=2, F=512, V=1000, P=300)


def draw(seed, vocab, n_prompts, plen_range, count_range, clen_range):
    """Seeded prompts and candidates: returns (ids for the call, prompt
    lengths, candidate lengths, counts, per-candidate full sequences)."""
    rng = np.random.default_rng(seed)
    plens = rng.integers(plen_range[0], plen_range[1] + 1, size=n_prompts).astype(np.int32)
    counts = rng.integers(count_range[0], count_range[1] + 1, size=n_prompts).astype(np.int32)
    prompts = [rng.integers(0, vocab, size=int(n)).astype(np.int32) for n in plens]
    cands, clens, full = [], [], []
    for p in range(n_prompts):
        for _ in range(int(counts[p])):
            c = rng.integers(0, vocab, size=int(rng.integers(clen_range[0], clen_range[1] + 1))).astype(np.int32)
            cands.append(c)
            clens.append(c.size)
            full.append(np.concatenate([prompts[p], c]))
    ids = np.concatenate(prompts + cands).astype(np.int32)
    return ids, plens, np.asarray(clens, np.int32), counts, full


def concatenated_rewards(torch, sc, full):
    lengths = np.array([s.size for s in full], dtype=np.int32)
    d = torch.from_numpy(np.concatenate(full)).cuda()
    r, _ = sc.score_requests(d, lengths, batch_overhead=64)
    torch.cuda.synchronize()
    return r.clone()


@pytest.mark.parametrize("cfg", [DEC64, DEC128], ids=["d64", "d128"])
@pytest.mark.parametrize("group,lanes", [(1, 1), (2, 2)])
def test_shared_prompts_bitwise_equal_concatenated(cfg, group, lanes):
    torch = need_gpu()
    w = make_weights(cfg)
    ids, plens, clens, counts, full = draw(3, cfg.vocab, 7, (1, 150), (1, 6), (1, 70))
    say(cfg.name, "prompts", plens.tolist(), "candidates", counts.tolist())
    sc = Scorer(blob.to_bytes(cfg, w, 0.25), 1200, 512)
    sc.set_attention("fused")
    want = concatenated_rewards(torch, sc, full)
    sc.set_grouping(group)
    sc.set_concurrency(lanes)
    d = torch.from_numpy(ids).cuda()
    for _ in range(2):
        rew, best, stats = sc.score_best_of_n(d, plens, clens, counts, batch_overhead=64)
        torch.cuda.synchronize()
        assert torch.equal(rew, want), float((rew - want).abs().max())
    assert stats["packed_tokens"] == int(plens.sum() + clens.sum())
    r = rew.cpu().numpy().astype(np.float64)
    assert best.cpu().numpy().tolist() == oracle.best_of_n(r.tolist(), counts.tolist())
    sc.set_pruning(False)                        # the full last layer: same bits
    full, _, _ = sc.score_best_of_n(d, plens, clens, counts, batch_overhead=64)
    torch.cuda.synchronize()
    assert torch.equal(full, rew)


@pytest.mark.parametrize("cfg", [DEC64, DEC128], ids=["d64", "d128"])
def test_shared_prompt_blocks_edge_cases(cfg):
    """Prompts just below, at and above the length from which candidates of
    a prompt share its key tiles four query tiles to a block (64), candidate
    lengths at the tile and block limits (1, 32, 33, 64, 65), and candidate
    counts that leave 1, 2 and 3 of a block's four slots filled: every
    reward bitwise equal to the prompt + candidate scored as one sequence."""
    torch = need_gpu()
    w = make_weights(cfg)
    rng = np.random.default_rng(31)
    plens = [63, 64, 65, 96, 130]
    clen_sets = [[1, 32], [33], [64, 65, 1], [32, 33, 64, 1, 2], [65, 64]]
    prompts = [rng.integers(0, cfg.vocab, size=n).astype(np.int32) for n in plens]
    cands, clens, counts, full = [], [], [], []
    for p, cl in zip(prompts, clen_sets):
        counts.append(len(cl))
        for n in cl:
            c = rng.integers(0, cfg.vocab, size=n).astype(np.int32)
            cands.append(c)
            clens.append(n)
            full.append(np.concatenate([p, c]))
    ids = np.concatenate(prompts + cands).astype(np.int32)
    sc = Scorer(blob.to_bytes(cfg, w, 0.0), 1200, 512)
    sc.set_attention("fused")
    want = concatenated_rewards(torch, sc, full)
    rew, best, _ = sc.score_best_of_n(torch.from_numpy(ids).cuda(), np.array(plens, np.int32),
                                      np.array(clens, np.int32), np.array(counts, np.int32),
                                      batch_overhead=64)
    torch.cuda.synchronize()
    assert torch.equal(rew, want), float((rew - want).abs().max())


def test_shared_prompts_match_oracle():
    torch = need_gpu()
    cfg = DEC64
    w = make_weights(cfg)
    ids, plens, clens, counts, full = draw(9, cfg.vocab, 4, (20, 120), (2, 4), (1, 50))
    sc = Scorer(blob.to_bytes(cfg, w, 0.0), 1200, 512)
    rew, best, _ = sc.score_best_of_n(torch.from_numpy(ids).cuda(), plens, clens, counts)
    torch.cuda.synchronize()
    got = rew.cpu().numpy().astype(np.float64)
    m = oracle.OracleModel(cfg, w)
    want = np.array([m.score(s) for s in full])
    say("best-of-n vs oracle: max |d| =", float(np.max(np.abs(got - want))))
    assert np.max(np.abs(got - want)) <= BF16_TOL
    assert best.cpu().numpy().tolist() == oracle.best_of_n(got.tolist(), counts.tolist())


def test_equal_candidates_pick_the_lowest_index():
    torch = need_gpu()
    cfg = DEC64
    w = make_weights(cfg)
    rng = np.random.default_rng(4)
    prompt = rng.integers(0, cfg.vocab, size=40).astype(np.int32)
    a = rng.integers(0, cfg.vocab, size=12).astype(np.int32)
    b = rng.integers(0, cfg.vocab, size=9).astype(np.int32)
    # candidates: b, a, a, b, a -- equal sequences get bitwise equal rewards
    cands = [b, a, a, b, a]
    ids = np.concatenate([prompt] + cands)
    sc = Scorer(blob.to_bytes(cfg, w, 0.0), 1200, 512)
    rew, best, _ = sc.score_best_of_n(torch.from_numpy(ids).cuda(), [40], [c.size for c in cands], [5])
    torch.cuda.synchronize()
    r = rew.cpu().numpy()
    assert r[1] == r[2] == r[4] and r[0] == r[3]
    assert int(best.cpu()[0]) == (1 if r[1] > r[0] else 0)


def test_best_of_n_validation():
    torch = need_gpu()
    w = make_weights(DEC64)
    sc = Scorer(blob.to_bytes(DEC64, w, 0.0), 200, 16)
    d = torch.zeros(400, dtype=torch.int32, device="cuda")
    bad = [
        (([10], [5, 5], [0]), -1),            # a prompt without candidates
        (([0], [5], [1]), -2),                # empty prompt
        (([10], [0], [1]), -2),               # empty candidate
        (([290], [20], [1]), -2),             # prompt + candidate above max_pos (300)
        (([150], [30, 30], [2]), -3),         # group of 210 tokens above max_tokens (200)
        (([5], [1] * 16, [16]), -3),          # 17 sequences above max_seqs (16)
    ]
    for (pl, cl, cc), status in bad:
        with pytest.raises(EncScoreError) as e:
            sc.score_best_of_n(d, pl, cl, cc)
        assert e.value.status == status, (pl, cl, cc, e.value.status)
    for cfg in (mini("enc", False, False, True, H=64, A=2, F=128, P=64),     # bidirectional
                mini("dec32", True, True, False, H=64, A=2, F=128, P=64)):   # fp32
        s2 = Scorer(blob.to_bytes(cfg, make_weights(cfg), 0.0), 200, 16)
        with pytest.raises(EncScoreError) as e:
            s2.score_best_of_n(d, [5], [5], [1])
        assert e.value.status == -1
