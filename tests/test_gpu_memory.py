"""Workspace memory modes (es_set_memory_mode) on the GPU.

TurboTransformers review, Proposed method: a sequence-length-aware allocator
keeps the intermediates' footprint low for variable-length inputs without
allocating per request.  Checks, through the C ABI:
  * rewards are bitwise the same with fixed workspaces, length-aware arenas
    and exact per-pass arenas (every model form, both attention forms,
    grouping, passes in flight, pruning on and off, shared prompts);
  * a length-aware arena is the size es_plan_arena gives for the pass's
    tensors (sizes from the pass's token count), rounded as documented;
  * steady state allocates nothing; a long call grows the arena and later
    short calls shrink it; exact mode allocates once per pass;
  * a bad mode is rejected.
"""
import numpy as np
import pytest

from encoder_scoring_amd import Scorer, blob
from helpers import mini, need_gpu, offsets_of, say
from oracle import memplan
from synth import get_config, make_weights
from synth.generate import random_stream

pytestmark = pytest.mark.gpu

MODELS = [
    ("enc_fp32_d26", mini("enc_fp32_d26", False, False, False, H=52, A=2, F=96, P=80)),
    ("enc_bf16", mini("enc_bf16", False, False, True, H=192, A=3, F=384, V=500, P=200)),
    ("dec_bf16_d128", mini("dec_bf16_d128", True, True, True, H=256, A=2, F=512, V=1000, P=300)),
    ("tinybert", get_config("tinybert")),
]
MiB = 1 << 20


def rewards(torch, sc, d, lengths, overhead=64):
    r, _ = sc.score_requests(d, lengths, batch_overhead=overhead)
    torch.cuda.synchronize()
    return r.clone()


@pytest.mark.parametrize("name,cfg", MODELS, ids=[m[0] for m in MODELS])
def test_memory_modes_give_bitwise_equal_rewards(name, cfg):
    torch = need_gpu()
    w = make_weights(cfg)
    ids, lengths = random_stream(31, 90, 1, min(cfg.max_pos, 120), cfg.vocab)
    d = torch.from_numpy(ids).cuda()
    sc = Scorer(blob.to_bytes(cfg, w, 0.25), 1500, 256)
    attentions = ["unfused", "fused"] if cfg.bf16 else ["unfused"]
    for att in attentions:
        if cfg.bf16:
            sc.set_attention(att)
        for group, lanes, prune in ((1, 1, True), (3, 2, True), (2, 1, False)):
            sc.set_grouping(group)
            sc.set_concurrency(lanes)
            sc.set_pruning(prune)
            got = {}
            for mode in ("fixed", "length_aware", "exact"):
                sc.set_memory_mode(mode)
                got[mode] = rewards(torch, sc, d, lengths)
                got[mode + "2"] = rewards(torch, sc, d, lengths)   # reuse of the same memory
            say(name, att, "group", group, "lanes", lanes, "prune", prune, sc.memory_stats())
            for k, v in got.items():
                assert torch.equal(v, got["fixed"]), (att, group, lanes, prune, k)
            # the single-batch entry point and es_forward_hidden too
            sc.set_memory_mode("fixed")
            off = offsets_of(lengths[:20])
            dd = d[: int(off[-1])]
            a = sc.score(dd, off).clone()
            ha = sc.hidden(dd, off).clone()
            sc.set_memory_mode("length_aware")
            b = sc.score(dd, off).clone()
            hb = sc.hidden(dd, off).clone()
            torch.cuda.synchronize()
            assert torch.equal(a, b) and torch.equal(ha, hb)


def test_shared_prompts_in_every_memory_mode():
    torch = need_gpu()
    cfg = MODELS[2][1]
    w = make_weights(cfg)
    rng = np.random.default_rng(2)
    plens = rng.integers(5, 120, size=6).astype(np.int32)
    counts = rng.integers(1, 5, size=6).astype(np.int32)
    clens = rng.integers(1, 60, size=int(counts.sum())).astype(np.int32)
    ids = rng.integers(0, cfg.vocab, size=int(plens.sum() + clens.sum())).astype(np.int32)
    d = torch.from_numpy(ids).cuda()
    sc = Scorer(blob.to_bytes(cfg, w, 0.0), 1200, 256)
    out = {}
    for mode in ("fixed", "length_aware", "exact"):
        sc.set_memory_mode(mode)
        r, b, _ = sc.score_best_of_n(d, plens, clens, counts, batch_overhead=64)
        torch.cuda.synchronize()
        out[mode] = (r.clone(), b.clone())
    for mode in ("length_aware", "exact"):
        assert torch.equal(out[mode][0], out["fixed"][0]) and torch.equal(out[mode][1], out["fixed"][1])


def pass_records(cfg, n_tokens, score_elems):
    """The workspace tensors of one pass and the steps that use them
    (0 embedding, 1 pre-LN LayerNorm, 2 QKV, 3 attention, 4 last-row gather,
    5 attention-out GEMM, 6 its LayerNorm, 7 FFN1, 8 FFN2, 9 FFN LayerNorm,
    10 head), sized from the pass's rows (tokens rounded up to 256)."""
    H, A, F = cfg.hidden, cfg.n_heads, cfg.ffn
    d = H // A
    dp = 32
    while dp < d:
        dp *= 2
    act = 2 if cfg.bf16 else 4
    up = lambda v, m: -(-v // m) * m
    rows = max(up(n_tokens, 256), 256)
    Hp, Kc, Fp, Nqkv = up(H, 64), up(A * dp, 64), up(F, 64), 3 * A * dp
    nb = [rows * H * 4, rows * Hp * act, rows * Nqkv * act, rows * Kc * act, rows * H * 4,
          rows * Fp * act, score_elems * 4, score_elems * act]
    return nb, [0, 0, 2, 3, 4, 7, 3, 3], [10, 10, 5, 5, 9, 8, 3, 3]


def test_arena_size_follows_the_pass():
    torch = need_gpu()
    cfg = get_config("tinybert")
    w = make_weights(cfg)
    sc = Scorer(blob.to_bytes(cfg, w, 0.0), 16384, 512)
    sc.set_attention("fused")
    base = sc.memory_stats()["device_bytes"]
    rng = np.random.default_rng(3)
    for n_seqs, length in ((3, 40), (64, 128), (40, 200)):
        lengths = np.full(n_seqs, length, dtype=np.int32)
        ids = rng.integers(0, cfg.vocab, size=int(lengths.sum())).astype(np.int32)
        d = torch.from_numpy(ids).cuda()
        sc.set_memory_mode("exact")                       # the arena is exactly this pass's need
        sc.score(d, offsets_of(lengths))
        torch.cuda.synchronize()
        nb, f, l = pass_records(cfg, int(lengths.sum()), 0)
        _, need = memplan.greedy_by_size(nb, f, l, 4096)
        st = sc.memory_stats()
        say("tokens", int(lengths.sum()), "need", need, st)
        assert st["work_bytes"] == need and st["device_bytes"] == base + need
        sc.set_memory_mode("length_aware")                # need + 1/8, in 16 MiB steps
        sc.score(d, offsets_of(lengths))
        torch.cuda.synchronize()
        assert sc.memory_stats()["work_bytes"] == -(-(need + need // 8) // (16 * MiB)) * 16 * MiB


def test_steady_state_growth_and_shrink():
    torch = need_gpu()
    cfg = MODELS[1][1]
    w = make_weights(cfg)
    sc = Scorer(blob.to_bytes(cfg, w, 0.0), 8192, 512)
    sc.set_attention("unfused")                           # score blocks live in the arena too
    short_ids, short_len = random_stream(4, 200, 1, 30, cfg.vocab)
    long_ids, long_len = random_stream(5, 300, 60, 100, cfg.vocab)
    ds, dl = torch.from_numpy(short_ids).cuda(), torch.from_numpy(long_ids).cuda()
    sc.set_memory_mode("fixed")
    fixed = sc.memory_stats()["work_bytes"]
    ref_s, ref_l = rewards(torch, sc, ds, short_len, 10**6), rewards(torch, sc, dl, long_len, 10**6)
    sc.set_memory_mode("length_aware")
    assert torch.equal(rewards(torch, sc, ds, short_len, 10**6), ref_s)
    small = sc.memory_stats(reset=True)["work_bytes"]
    assert torch.equal(rewards(torch, sc, ds, short_len, 10**6), ref_s)
    assert sc.memory_stats()["allocs"] == 0               # steady state: no allocation
    assert torch.equal(rewards(torch, sc, dl, long_len, 10**6), ref_l)
    big = sc.memory_stats()["work_bytes"]
    assert big > 2 * small and big < fixed
    for _ in range(2):                                    # the next short call shrinks it
        assert torch.equal(rewards(torch, sc, ds, short_len, 10**6), ref_s)
    after = sc.memory_stats()["work_bytes"]
    say("fixed", fixed, "short", small, "long", big, "after", after)
    assert after < big and after <= 2 * small
    sc.set_memory_mode("exact")
    sc.memory_stats(reset=True)
    _, st = sc.score_requests(ds, short_len, batch_overhead=10**6)
    torch.cuda.synchronize()
    assert sc.memory_stats()["allocs"] == st["n_batches"]  # one arena per pass (grouping 1)


def test_bad_memory_mode():
    need_gpu()
    cfg = MODELS[0][1]
    sc = Scorer(blob.to_bytes(cfg, make_weights(cfg), 0.0), 256, 16)
    with pytest.raises(KeyError):
        sc.set_memory_mode("bogus")
    assert sc.lib.es_set_memory_mode(sc.handle, 7) == -1       # ES_ERR_ARG
    assert b"memory mode 7" in sc.lib.es_last_error()
