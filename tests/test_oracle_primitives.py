"""Pins for the oracle's row primitives: closed forms, textbook values, hand examples.

None of these re-types the oracle's formula: each checks a property or value
fixed by mathematics (row sums, moments, Phi tables, worked examples) or by an
independent library routine.
"""
import json
import math
import os

import numpy as np
import pytest

from oracle import attention, gelu, layer_norm, masked_attention, softmax_rows

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _hand():
    with open(os.path.join(GOLD, "hand_examples.json")) as f:
        return json.load(f)


# ---------------------------------------------------------------- softmax

@pytest.mark.parametrize("dtype,tol", [(np.float64, 1e-13), (np.float32, 1e-6)])
def test_softmax_rows_sum_to_one(dtype, tol):
    rng = np.random.default_rng(0)
    s = (rng.standard_normal((37, 53)) * 5).astype(dtype)   # non-square: wrong axis fails
    p = softmax_rows(s)
    assert p.dtype == dtype
    assert np.all(p >= 0)
    np.testing.assert_allclose(p.sum(axis=1), 1.0, atol=tol)


def test_softmax_closed_forms():
    h = _hand()["softmax"]
    np.testing.assert_allclose(softmax_rows(np.array([h["row"]])), [h["p"]], atol=1e-15)
    for m in (1, 2, 4, 64, 512):
        p = softmax_rows(np.full((3, m), 0.7))
        assert np.all(p == 1.0 / m)                     # exact for powers of two
    assert softmax_rows(np.array([[123.0]]))[0, 0] == 1.0


def test_softmax_shift_invariance_and_large_values():
    rng = np.random.default_rng(1)
    s = rng.standard_normal((5, 40))
    np.testing.assert_allclose(softmax_rows(s), softmax_rows(s + 1000.0), atol=1e-12)
    assert np.all(np.isfinite(softmax_rows(s * 1e3)))   # max subtraction present


def test_softmax_masked_entries_get_zero():
    s = np.array([[1.0, -np.inf, 2.0, -np.inf]])
    p = softmax_rows(s)
    assert p[0, 1] == 0.0 and p[0, 3] == 0.0
    np.testing.assert_allclose(p[0, [0, 2]], [1 / (1 + math.e), math.e / (1 + math.e)], atol=1e-15)


# ---------------------------------------------------------------- layernorm

@pytest.mark.parametrize("n", [4, 5, 128, 312, 768])
def test_layernorm_moments(n):
    rng = np.random.default_rng(n)
    x = rng.standard_normal((9, n)) * 0.02 + 0.3
    eps = 1e-12
    z = layer_norm(x, np.ones(n), np.zeros(n), eps)
    np.testing.assert_allclose(z.mean(axis=1), 0.0, atol=1e-12)
    var = x.var(axis=1)                                # biased (numpy default ddof=0)
    np.testing.assert_allclose(z.var(axis=1), var / (var + eps), atol=1e-9)


def test_layernorm_hand_example_and_affine():
    h = _hand()["layer_norm"]
    x = np.array([h["x"]])
    np.testing.assert_allclose(layer_norm(x, np.ones(4), np.zeros(4), 0.0), [h["z"]], atol=1e-14)
    np.testing.assert_allclose(layer_norm(x, np.full(4, 2.0), np.ones(4), 0.0),
                               [h["y_gain2_shift1"]], atol=1e-14)


def test_layernorm_constant_row_gives_shift():
    g = np.linspace(0.5, 2.0, 16)
    b = np.linspace(-1.0, 1.0, 16)
    y = layer_norm(np.full((2, 16), 0.5), g, b, 1e-12)
    assert np.array_equal(y, np.broadcast_to(b, y.shape))


def test_layernorm_eps_enters_under_root():
    x = np.array([[1.0, -1.0]])                        # var = 1
    z = layer_norm(x, np.ones(2), np.zeros(2), 3.0)
    np.testing.assert_allclose(z, [[0.5, -0.5]], atol=1e-15)   # 1 / sqrt(1 + 3)


# ---------------------------------------------------------------- gelu

def _phi_table():
    rows = []
    with open(os.path.join(GOLD, "normal_cdf.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                a, b = line.split()
                rows.append((float(a), float(b)))
    return rows


def test_gelu_matches_normal_table():
    for x, phi in _phi_table():
        assert abs(float(gelu(np.array(x))) - x * phi) < 1e-10, x


def test_gelu_identities():
    x = np.linspace(-6, 6, 241)
    np.testing.assert_allclose(gelu(x) - gelu(-x), x, atol=1e-14)   # x*Phi(x) + x*Phi(-x) = x
    assert float(gelu(np.array(0.0))) == 0.0
    assert gelu(np.float32(np.ones(3))).dtype == np.float32
    # tanh approximation differs by ~1e-4 near |x| = 2: the exact form is used
    tanh_form = 0.5 * 2.0 * (1 + math.tanh(math.sqrt(2 / math.pi) * (2.0 + 0.044715 * 8.0)))
    assert abs(float(gelu(np.array(2.0))) - tanh_form) > 1e-5


# ---------------------------------------------------------------- attention

def test_attention_hand_example():
    h = _hand()["attention_1d"]
    x = np.array(h["x"]).reshape(2, 1)
    w = np.ones((3, 1))
    b = np.zeros(3)
    np.testing.assert_allclose(attention(x, w, b, 1, False)[:, 0], h["ctx_bidirectional"], atol=1e-14)
    np.testing.assert_allclose(attention(x, w, b, 1, True)[:, 0], h["ctx_causal"], atol=1e-14)


def test_attention_single_token_returns_value():
    rng = np.random.default_rng(3)
    H, A = 24, 3
    x = rng.standard_normal((1, H))
    w = rng.standard_normal((3 * H, H))
    b = rng.standard_normal(3 * H)
    v = x @ w[2 * H:].T + b[2 * H:]
    for causal in (False, True):
        np.testing.assert_allclose(attention(x, w, b, A, causal), v, atol=1e-13)


def test_attention_zero_query_gives_means():
    rng = np.random.default_rng(4)
    n, H, A = 7, 12, 3
    x = rng.standard_normal((n, H))
    w = rng.standard_normal((3 * H, H))
    b = rng.standard_normal(3 * H)
    w[:H] = 0.0
    b[:H] = 0.0                                   # all scores 0 -> uniform weights
    v = x @ w[2 * H:].T + b[2 * H:]
    np.testing.assert_allclose(attention(x, w, b, A, False), np.broadcast_to(v.mean(0), v.shape), atol=1e-13)
    prefix = np.cumsum(v, axis=0) / np.arange(1, n + 1)[:, None]
    np.testing.assert_allclose(attention(x, w, b, A, True), prefix, atol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_masked_attention_matches_torch_sdpa(causal):
    """Independent implementation on given Q, K, V: torch's
    scaled_dot_product_attention on the CPU (float64), heads split from the
    concatenated columns."""
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(6)
    n, A, d = 37, 3, 8
    q, k, v = (rng.standard_normal((n, A * d)) for _ in range(3))
    heads = lambda a: torch.from_numpy(a.reshape(n, A, d).transpose(1, 0, 2).copy())
    ref = torch.nn.functional.scaled_dot_product_attention(heads(q), heads(k), heads(v), is_causal=causal)
    ref = ref.numpy().transpose(1, 0, 2).reshape(n, A * d)
    np.testing.assert_allclose(masked_attention(q, k, v, A, causal), ref, atol=1e-12)


def test_masked_attention_dominant_key():
    """A key whose score exceeds every other by 60 takes all the weight: each
    query's context is that key's value row (to exp(-60))."""
    n, H = 6, 4
    rng = np.random.default_rng(7)
    v = rng.standard_normal((n, H))
    q = np.zeros((n, H)); q[:, 0] = 1.0
    k = np.zeros((n, H)); k[2, 0] = 120.0          # score 120 / sqrt(4) = 60
    ctx = masked_attention(q, k, v, 1, False)
    np.testing.assert_allclose(ctx, np.broadcast_to(v[2], (n, H)), atol=1e-20 + 1e-24)
    causal = masked_attention(q, k, v, 1, True)   # rows 0, 1 cannot see key 2
    np.testing.assert_allclose(causal[2:], np.broadcast_to(v[2], (n - 2, H)), atol=1e-20)
    np.testing.assert_allclose(causal[1], v[:2].mean(0), atol=1e-14)


@pytest.mark.parametrize("causal", [False, True])
def test_attention_matches_torch_multihead(causal):
    """Independent implementation: torch.nn.MultiheadAttention on the CPU (float64)."""
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(5)
    n, H, A = 11, 24, 4
    x = rng.standard_normal((n, H))
    w = rng.standard_normal((3 * H, H)) * 0.3
    b = rng.standard_normal(3 * H) * 0.3
    mha = torch.nn.MultiheadAttention(H, A, bias=True, batch_first=True, dtype=torch.float64)
    with torch.no_grad():
        mha.in_proj_weight.copy_(torch.from_numpy(w))
        mha.in_proj_bias.copy_(torch.from_numpy(b))
        mha.out_proj.weight.copy_(torch.eye(H, dtype=torch.float64))
        mha.out_proj.bias.zero_()
    mask = torch.triu(torch.ones(n, n, dtype=torch.bool), 1) if causal else None
    xt = torch.from_numpy(x)[None]
    with torch.no_grad():
        ref = mha(xt, xt, xt, attn_mask=mask, need_weights=False)[0][0].numpy()
    np.testing.assert_allclose(attention(x, w, b, A, causal), ref, atol=1e-12)
