"""CPU checks of the per-pass metadata the library builds on the host
(es_check_plan): for every workload's full plan -- grouping of planned
batches into passes, shared prompts -- every token offset, id source, reward
slot, score-block base, softmax row address and attention / softmax /
last-token work item indexes inside the buffer it addresses, and every query
tile and score row is covered exactly once."""
import ctypes

import numpy as np
import pytest

from bench import DEFAULT_GROUP, LAUNCH

# every grouping a timed configuration uses, and the edges
GROUPS = sorted({1, 2, DEFAULT_GROUP, 8} | {g for g, _ in LAUNCH.values()})
from encoder_scoring_amd import _lib, blob, check_plan
from encoder_scoring_amd._lib import ES_ERR_CAPACITY, ES_ERR_FORMAT, ES_ERR_RANGE, EncScoreError
from synth import get_config, make_fixed_batch, make_requests, make_weights
from synth.configs import ORDERED
from synth.generate import best_of_n_form


def _shape(cfg):
    return dict(n_heads=cfg.n_heads, causal=cfg.causal, max_pos=cfg.max_pos,
                max_tokens=cfg.max_tokens, max_seqs=min(cfg.max_tokens, 65536))


@pytest.mark.parametrize("group", GROUPS)
@pytest.mark.parametrize("name", ORDERED)
def test_every_workload_plan_indexes_inside_its_buffers(name, group):
    cfg = get_config(name)
    if name == "tinybert":
        _, lengths = make_fixed_batch(cfg, 256, 64)
    else:
        _, lengths, _ = make_requests(cfg)
    passes, checked, bad = check_plan(lengths, batch_overhead=cfg.batch_overhead,
                                      batches_per_pass=group, **_shape(cfg))
    assert bad == 0 and passes >= 1 and checked > 100 * lengths.size


@pytest.mark.parametrize("group", sorted(set(GROUPS) - {2}))
def test_shared_prompt_plan_indexes_inside_its_buffers(group):
    cfg = get_config("decoder_rm")
    ids, lengths, grp = make_requests(cfg)
    _, pl, _, cl, cn = best_of_n_form(ids, lengths, grp, 512)
    passes, checked, bad = check_plan(cl, batch_overhead=cfg.batch_overhead, batches_per_pass=group,
                                      prompt_lengths=pl, cand_counts=cn, **_shape(cfg))
    assert bad == 0 and passes >= 1 and checked > 1000


def test_random_plans_index_inside_their_buffers():
    rng = np.random.default_rng(17)
    for _ in range(300):
        n = int(rng.integers(1, 60))
        P = int(rng.integers(8, 600))
        lengths = rng.integers(1, P + 1, size=n)
        T = int(rng.integers(P, 4 * P + 1))
        A, causal = int(rng.integers(1, 17)), bool(rng.integers(0, 2))
        _, _, bad = check_plan(lengths, A, causal, P, T, T, int(rng.integers(0, 300)),
                               int(rng.integers(1, 6)))
        assert bad == 0
        if causal:  # the same requests as prompt + candidate groups
            k = int(rng.integers(1, 5))
            counts = rng.integers(1, 6, size=k)
            plen = rng.integers(1, max(2, P // 2), size=k)
            cand = np.concatenate([rng.integers(1, P - p + 1, size=c) for p, c in zip(plen, counts)])
            _, _, bad = check_plan(cand, A, True, P, max(T, int((plen + P).max()) * 4), 64,
                                   int(rng.integers(0, 300)), int(rng.integers(1, 4)),
                                   prompt_lengths=plen, cand_counts=counts)
            assert bad == 0


@pytest.mark.parametrize("lengths,code", [([3, 70], ES_ERR_RANGE), ([0, 2], ES_ERR_RANGE),
                                          ([64] * 5, None)])
def test_plan_validation(lengths, code):
    if code is None:  # fits: 64-token sequences, budget 128 tokens per batch
        assert check_plan(lengths, 2, True, 64, 128, 8, 4, 1)[2] == 0
        return
    with pytest.raises(EncScoreError) as e:
        check_plan(lengths, 2, True, 64, 128, 8, 4, 1)
    assert e.value.status == code


def test_stream_batch_over_max_seqs_is_refused():
    # the planner fills a 64-token budget with 64 one-token requests; the
    # handle holds 8 sequences per batch
    with pytest.raises(EncScoreError) as e:
        check_plan([1] * 64, 2, False, 64, 64, 8, 0, 1)
    assert e.value.status == ES_ERR_CAPACITY


def test_shared_prompt_group_over_capacity_is_refused():
    with pytest.raises(EncScoreError) as e:  # one prompt group of 120 tokens, budget 64
        check_plan([40, 40], 2, True, 100, 64, 8, 4, 1, prompt_lengths=[40], cand_counts=[2])
    assert e.value.status == ES_ERR_CAPACITY


def test_blob_info_reports_the_shape_and_rejects_corruption():
    lib = _lib.load()
    for name in ("tiny_fp32", "tinybert"):
        cfg = get_config(name)
        data = blob.to_bytes(cfg, make_weights(cfg), 0.25)
        info = _lib.ModelInfo()
        buf = ctypes.create_string_buffer(data, len(data))
        assert lib.es_blob_info(ctypes.cast(buf, ctypes.c_void_p), len(data), ctypes.byref(info)) == 0
        assert (info.n_layers, info.hidden, info.n_heads, info.ffn, info.vocab, info.max_pos) == \
            (cfg.n_layers, cfg.hidden, cfg.n_heads, cfg.ffn, cfg.vocab, cfg.max_pos)
        assert (bool(info.bf16), bool(info.causal), info.reward_offset) == (cfg.bf16, cfg.causal, 0.25)
        assert lib.es_blob_info(ctypes.cast(buf, ctypes.c_void_p), len(data) - 1,
                                ctypes.byref(info)) == ES_ERR_FORMAT
