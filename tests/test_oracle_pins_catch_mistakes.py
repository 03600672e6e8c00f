"""Plant plausible mistakes in the oracle (on the CPU) and show a pin catches each.

Each mutant replaces one oracle primitive for the duration of the test; the
independent torch reference or an invariant must then disagree.
"""
import math

import numpy as np
import pytest

import oracle.model as om
from oracle import OracleModel
from synth import make_weights
from synth.generate import random_stream, split
from test_oracle_model import MINIS, torch_reference


def _max_torch_gap(cfg, n_seq=3):
    w = make_weights(cfg)
    ids, lengths = random_stream(21, n_seq, 2, 20, cfg.vocab)
    m = OracleModel(cfg, w)
    return max(abs(m.score(s) - torch_reference(cfg, w, s)) for s in split(ids, lengths))


def _ln_unbiased(x, g, b, eps):
    mu = x.mean(axis=-1, keepdims=True)
    var = x.var(axis=-1, keepdims=True, ddof=1)
    return (x - mu) / np.sqrt(var + eps) * g + b


def _gelu_tanh(z):
    z = np.asarray(z)
    return 0.5 * z * (1 + np.tanh(math.sqrt(2 / math.pi) * (z + 0.044715 * z ** 3)))


def _attention_kt_swapped(x, w_qkv, b_qkv, n_heads, causal, key_mask=None):
    # K and V blocks exchanged
    H = x.shape[1]
    w = np.concatenate([w_qkv[:H], w_qkv[2 * H:], w_qkv[H:2 * H]])
    b = np.concatenate([b_qkv[:H], b_qkv[2 * H:], b_qkv[H:2 * H]])
    return ORIG["attention"](x, w, b, n_heads, causal, key_mask)


ORIG = {"attention": om.attention, "layer_norm": om.layer_norm, "gelu": om.gelu}


@pytest.mark.parametrize("name,mutant", [
    ("layer_norm", _ln_unbiased),
    ("attention", _attention_kt_swapped),
])
def test_torch_pin_detects_mutant(monkeypatch, name, mutant):
    cfg = MINIS[0]
    assert _max_torch_gap(cfg) < 1e-10
    monkeypatch.setattr(om, name, mutant)
    assert _max_torch_gap(cfg) > 1e-7


def test_causal_pin_detects_missing_mask(monkeypatch):
    cfg = MINIS[2]
    assert _max_torch_gap(cfg) < 1e-10
    orig = om.attention
    monkeypatch.setattr(om, "attention",
                        lambda x, w, b, A, causal, key_mask=None: orig(x, w, b, A, False, key_mask))
    assert _max_torch_gap(cfg) > 1e-7


def test_head_on_first_token_detected(monkeypatch):
    cfg = MINIS[0]
    monkeypatch.setattr(OracleModel, "score",
                        lambda self, ids, offset=0.0: float(self.head(self.hidden(ids)[:1], offset)[0]))
    assert _max_torch_gap(cfg) > 1e-7


def test_packed_pin_detects_global_positions(monkeypatch):
    """If positions did not restart per sequence, packed != one-at-a-time."""
    cfg = MINIS[0]
    m = OracleModel(cfg, make_weights(cfg))
    ids, lengths = random_stream(22, 3, 3, 9, cfg.vocab)
    good = m.score_many(split(ids, lengths))
    orig_embed = OracleModel.embed
    monkeypatch.setattr(OracleModel, "embed",
                        lambda self, i, p: orig_embed(self, i, np.arange(len(i))))
    bad = m.score_packed(ids, lengths)
    assert np.max(np.abs(bad - good)) > 1e-6


def test_phi_table_pin_detects_tanh_gelu():
    """At N(0, 0.02) weights the FFN inputs are small, so the whole-model gap
    of a tanh-form GELU is tiny; the textbook Phi table catches it directly."""
    from test_oracle_primitives import _phi_table
    worst = max(abs(float(_gelu_tanh(np.array(x))) - x * phi) for x, phi in _phi_table())
    assert worst > 1e-5
    worst_exact = max(abs(float(om.gelu(np.array(x))) - x * phi) for x, phi in _phi_table())
    assert worst_exact < 1e-10


def test_selection_pins_detect_ties_to_the_last_index(monkeypatch):
    """A best-of-N that lets an equal later reward win (>= instead of >) must
    fail the hand-worked tie cases."""
    import json
    import os
    import oracle.selection as sel

    def last_wins(rewards, counts):
        out, start = [], 0
        for c in counts:
            k = 0
            for j in range(1, c):
                if rewards[start + j] >= rewards[start + k]:
                    k = j
            out.append(k)
            start += c
        return out

    golden = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "hand_examples.json")))
    monkeypatch.setattr(sel, "best_of_n", last_wins)
    assert any(sel.best_of_n(c["rewards"], c["counts"]) != c["best"] for c in golden["best_of_n"])
