"""The allocation-free entry point es_score_batch_static, through the C ABI.

It runs es_score_batch's kernels with every intermediate in the library's
fixed per-GPU scratch array, so its rewards must be bitwise those of
es_score_batch on the same handle and inputs.  Checked on two calls in a row,
the second with a smaller batch (the array keeps the first call's contents),
for an fp32 encoder and bf16 encoder / causal decoder models in both
attention forms; the handle's own workspace must stay unallocated while only
the static entry point runs; a batch needing more than the array is refused
with ES_ERR_CAPACITY before any device work.
"""
import numpy as np
import pytest

from encoder_scoring_amd import EncScoreError, Scorer, blob
from encoder_scoring_amd._lib import ES_ERR_CAPACITY
from helpers import mini, need_gpu, offsets_of, say
from synth import get_config, make_weights
from synth.generate import random_stream

pytestmark = pytest.mark.gpu

CASES = [
    ("tiny_fp32", get_config("tiny_fp32"), "unfused"),
    ("enc_bf16", mini("enc_bf16", False, False, True, H=192, A=3, F=384, V=500, P=200), "unfused"),
    ("enc_bf16", mini("enc_bf16", False, False, True, H=192, A=3, F=384, V=500, P=200), "fused"),
    ("dec_bf16", mini("dec_bf16", True, True, True, H=256, A=2, F=512, V=1000, P=300), "unfused"),
    ("dec_bf16", mini("dec_bf16", True, True, True, H=256, A=2, F=512, V=1000, P=300), "fused"),
]


@pytest.mark.parametrize("name,cfg,attention", CASES, ids=[f"{c[0]}-{c[2]}" for c in CASES])
def test_static_matches_score_batch_twice(name, cfg, attention):
    torch = need_gpu()
    w = make_weights(cfg)
    sc = Scorer(blob.to_bytes(cfg, w, 0.0625), 8192, 512)
    sc.set_attention(attention)
    big_ids, big_len = random_stream(41, 37, 1, min(cfg.max_pos, 200), cfg.vocab)
    small_ids, small_len = random_stream(42, 5, 1, min(cfg.max_pos, 60), cfg.vocab)
    got = []
    for ids, lengths in ((big_ids, big_len), (small_ids, small_len)):
        d = torch.from_numpy(ids).cuda()
        out = torch.full((lengths.size,), float("nan"), dtype=torch.float32, device="cuda")
        sc.score_static(d, offsets_of(lengths), out)
        torch.cuda.synchronize()
        got.append(out.cpu().numpy())
    st = sc.memory_stats()
    say(name, attention, "after static calls:", st)
    assert st["allocs"] == 0 and st["work_bytes"] == 0   # the handle's workspace never allocated
    for (ids, lengths), g in zip(((big_ids, big_len), (small_ids, small_len)), got):
        want = sc.score(torch.from_numpy(ids).cuda(), offsets_of(lengths))
        torch.cuda.synchronize()
        assert np.array_equal(g, want.cpu().numpy()), f"{name} {attention}: {len(lengths)} sequences"
    # once more after the ordinary path ran in between
    d = torch.from_numpy(small_ids).cuda()
    out = torch.empty(small_len.size, dtype=torch.float32, device="cuda")
    sc.score_static(d, offsets_of(small_len), out)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy(), got[1])
    sc.close()


def test_static_refuses_a_batch_beyond_the_array():
    torch = need_gpu()
    cfg = mini("dec_big", True, True, True, H=512, A=4, F=2048, V=1000, P=512)
    sc = Scorer(blob.to_bytes(cfg, make_weights(cfg), 0.0), 65536, 512)
    lengths = np.full(100, 500, dtype=np.int32)       # 50k tokens: hundreds of MB of activations
    d = torch.zeros(int(lengths.sum()), dtype=torch.int32, device="cuda")
    out = torch.full((lengths.size,), 7.0, dtype=torch.float32, device="cuda")
    with pytest.raises(EncScoreError) as e:
        sc.score_static(d, offsets_of(lengths), out)
    assert e.value.status == ES_ERR_CAPACITY
    torch.cuda.synchronize()
    assert bool((out == 7.0).all().item())            # nothing ran
    sc.close()
