"""Pins for the oracle's whole forward pass.

* an independent third-party implementation: torch.nn.TransformerEncoderLayer
  (post-LN and pre-LN forms, exact-erf GELU) on the CPU in float64;
* invariants: packed, padded and one-at-a-time runs agree; permuting the
  batch permutes the rewards; calibrated reference rewards average zero;
* precision: the float32 oracle stays within 1e-5 of the float64 oracle.
"""
import numpy as np
import pytest

from oracle import OracleModel
from synth import get_config, make_weights, make_reference_set, make_requests
from synth.configs import ModelConfig
from synth.generate import random_stream, split, as_float


def mini(name, pre_ln, causal, bf16, H=64, A=4, F=128, L=2, V=97, P=48, eps=1e-5, seed=7):
    return ModelConfig(name=name, n_layers=L, hidden=H, n_heads=A, ffn=F, vocab=V, max_pos=P,
                       pre_ln=pre_ln, causal=causal, bf16=bf16, eps=eps,
                       seeds={"weights": seed, "requests": seed + 1, "reference": seed + 2})


MINIS = [
    mini("enc_fp32", False, False, False),
    mini("enc_bf16_d26", False, False, True, H=78, A=3, F=160, eps=1e-12),
    mini("dec_bf16", True, True, True),
    mini("dec_fp32_bidir", True, False, False),
]


def torch_reference(cfg, w, seq):
    """Score one sequence with torch.nn.TransformerEncoderLayer stacks (float64)."""
    torch = pytest.importorskip("torch")
    f = lambda name: torch.from_numpy(as_float(w[name], np.float64))
    H = cfg.hidden
    ids = torch.from_numpy(np.asarray(seq, dtype=np.int64))
    x = f("tok_emb")[ids] + f("pos_emb")[: len(seq)]
    if not cfg.pre_ln:
        x = torch.nn.functional.layer_norm(x, (H,), f("norm_g"), f("norm_b"), cfg.eps)
    x = x[None]
    mask = None
    if cfg.causal:
        mask = torch.triu(torch.ones(len(seq), len(seq), dtype=torch.bool), 1)
    for l in range(cfg.n_layers):
        p = f"l{l}."
        layer = torch.nn.TransformerEncoderLayer(
            H, cfg.n_heads, cfg.ffn, dropout=0.0, activation="gelu", layer_norm_eps=cfg.eps,
            batch_first=True, norm_first=cfg.pre_ln, dtype=torch.float64)
        layer.eval()
        with torch.no_grad():
            layer.self_attn.in_proj_weight.copy_(f(p + "w_qkv"))
            layer.self_attn.in_proj_bias.copy_(f(p + "b_qkv"))
            layer.self_attn.out_proj.weight.copy_(f(p + "w_o"))
            layer.self_attn.out_proj.bias.copy_(f(p + "b_o"))
            layer.linear1.weight.copy_(f(p + "w_1"))
            layer.linear1.bias.copy_(f(p + "b_1"))
            layer.linear2.weight.copy_(f(p + "w_2"))
            layer.linear2.bias.copy_(f(p + "b_2"))
            layer.norm1.weight.copy_(f(p + "ln1_g"))
            layer.norm1.bias.copy_(f(p + "ln1_b"))
            layer.norm2.weight.copy_(f(p + "ln2_g"))
            layer.norm2.bias.copy_(f(p + "ln2_b"))
            x = layer(x, src_mask=mask)
    h = x[0, -1]
    if cfg.pre_ln:
        h = torch.nn.functional.layer_norm(h, (H,), f("norm_g"), f("norm_b"), cfg.eps)
    return float(h @ f("head_w") + f("head_b")[0])


@pytest.mark.parametrize("cfg", MINIS, ids=lambda c: c.name)
def test_forward_matches_torch_encoder_layers(cfg):
    w = make_weights(cfg)
    ids, lengths = random_stream(11, 5, 1, cfg.max_pos, cfg.vocab)
    m = OracleModel(cfg, w)
    for s in split(ids, lengths):
        assert abs(m.score(s) - torch_reference(cfg, w, s)) < 1e-10


def test_forward_matches_torch_tiny_workload():
    cfg = get_config("tiny_fp32")
    w = make_weights(cfg)
    ids, lengths, _ = make_requests(cfg)
    m = OracleModel(cfg, w)
    for s in split(ids, lengths)[:4]:
        assert abs(m.score(s) - torch_reference(cfg, w, s)) < 1e-10


@pytest.mark.parametrize("cfg", MINIS, ids=lambda c: c.name)
def test_packed_padded_one_at_a_time_agree(cfg):
    w = make_weights(cfg)
    ids, lengths = random_stream(12, 6, 1, 30, cfg.vocab)
    seqs = split(ids, lengths)
    m = OracleModel(cfg, w)
    one = m.score_many(seqs, 0.25)
    np.testing.assert_allclose(m.score_packed(ids, lengths, 0.25), one, atol=1e-12)
    np.testing.assert_allclose(m.score_padded(seqs, 0.25), one, atol=1e-12)
    m32 = OracleModel(cfg, w, dtype=np.float32)
    np.testing.assert_allclose(m32.score_packed(ids, lengths), m32.score_many(seqs), atol=1e-6)


def test_permutation_equivariance():
    cfg = MINIS[2]
    w = make_weights(cfg)
    ids, lengths = random_stream(13, 7, 1, 25, cfg.vocab)
    seqs = split(ids, lengths)
    m = OracleModel(cfg, w)
    base = m.score_packed(ids, lengths)
    perm = np.random.default_rng(0).permutation(len(seqs))
    pseqs = [seqs[i] for i in perm]
    got = m.score_packed(np.concatenate(pseqs), lengths[perm])
    np.testing.assert_allclose(got, base[perm], atol=1e-12)


def test_positions_restart_per_sequence():
    """Two identical sequences packed together get identical rewards."""
    cfg = MINIS[0]
    m = OracleModel(cfg, make_weights(cfg))
    s = np.array([5, 9, 2, 44, 3], dtype=np.int32)
    r = m.score_packed(np.concatenate([s, s]), [5, 5])
    assert r[0] == pytest.approx(r[1], abs=1e-13)
    assert r[0] == pytest.approx(m.score(s), abs=1e-12)


@pytest.mark.parametrize("name", ["tiny_fp32"])
def test_reference_rewards_average_zero(name):
    cfg = get_config(name)
    m = OracleModel(cfg, make_weights(cfg))
    rid, rlen = make_reference_set(cfg)
    ref = split(rid, rlen)
    off = m.calibrate_offset(ref)
    assert abs(m.score_many(ref, off).mean()) < 1e-7   # offset stored as float32
    assert abs(off) > 1e-4                              # nontrivial offset


def test_float32_oracle_close_to_float64():
    cfg = get_config("tiny_fp32")
    w = make_weights(cfg)
    ids, lengths, _ = make_requests(cfg)
    seqs = split(ids, lengths)
    r64 = OracleModel(cfg, w).score_many(seqs)
    r32 = OracleModel(cfg, w, dtype=np.float32).score_many(seqs)
    assert np.max(np.abs(r64 - r32)) < 1e-5


def test_later_tokens_do_not_change_causal_prefix():
    """Causal decoder: the hidden state of a prefix ignores what follows it."""
    cfg = MINIS[2]
    m = OracleModel(cfg, make_weights(cfg))
    s = np.arange(20) % cfg.vocab
    h_full = m.hidden(s)
    h_pre = m.hidden(s[:12])
    np.testing.assert_allclose(h_full[:12], h_pre, atol=1e-12)


def test_bidirectional_later_tokens_do_change_scores():
    cfg = MINIS[0]
    m = OracleModel(cfg, make_weights(cfg))
    s = np.arange(20) % cfg.vocab
    assert abs(m.hidden(s)[11, 0] - m.hidden(s[:12])[11, 0]) > 1e-6
