"""Fused masked attention (es_op_attention) on the GPU against the oracle's
masked attention (float64 on the host, on the same bf16 Q, K, V values).

TurboTransformers review, Proposed method: the scores, their Softmax row
reduction and the context product of the encoder's attention; here in one
pass per query tile (short sequences: one wavefront per 32 queries; longer
ones: four query tiles per block sharing each key tile through LDS).

Tolerance per element: the kernel rounds the probabilities to bf16 before
the context product (each weight within 2^-9 relative) and the context to
bf16 (2^-9 relative); with fp32 accumulation otherwise,
    |ctx - exact| <= 2^-9 (max |V| + |exact|) + O(fp32),
so the bar is 4e-3 (max |V| of the head + |exact|), twice that bound.
"""
import numpy as np
import pytest

import oracle
from encoder_scoring_amd import EncScoreError, RaggedScores, attention_fused
from helpers import f32_to_bf16_bits, need_gpu, say

pytestmark = pytest.mark.gpu


def bits_to_f32(a):
    """uint16 / int16 numpy array of bf16 bit patterns -> float32."""
    return (np.ascontiguousarray(a).view(np.uint16).astype(np.uint32) << 16).view(np.float32)


def run_case(torch, lengths, n_heads, d, causal, q, k, v, ld_extra=8):
    """Pack q, k, v ([T, n_heads * d] float32, already bf16 values) as one
    Q | K | V buffer, run the op, return the context as float64 [T, H]."""
    T, H = q.shape
    ld = 3 * H + ld_extra
    qkv = np.zeros((T, ld), dtype=np.uint16)
    qkv[:, :H] = f32_to_bf16_bits(q)
    qkv[:, H:2 * H] = f32_to_bf16_bits(k)
    qkv[:, 2 * H:3 * H] = f32_to_bf16_bits(v)
    dq = torch.from_numpy(qkv.view(np.int16)).cuda()
    ldc = H + 4
    ctx = torch.full((T, ldc), 0x7abc, dtype=torch.int16, device="cuda")
    rag = RaggedScores(lengths, n_heads, causal)
    attention_fused(rag, dq, ctx, d)
    torch.cuda.synchronize()
    out = ctx.cpu().numpy()
    assert np.all(out[:, H:].view(np.uint16) == 0x7abc)             # columns past H untouched
    rag.close()
    return bits_to_f32(out[:, :H]).astype(np.float64)


def check_against_oracle(got, lengths, n_heads, causal, q, k, v):
    H = q.shape[1]
    d = H // n_heads
    worst = 0.0
    t0 = 0
    for n in lengths:
        sl = slice(t0, t0 + n)
        want = oracle.masked_attention(q[sl].astype(np.float64), k[sl].astype(np.float64),
                                       v[sl].astype(np.float64), n_heads, causal)
        for h in range(n_heads):
            cols = slice(h * d, (h + 1) * d)
            vmax = float(np.max(np.abs(v[sl, cols])))
            err = np.abs(got[sl, cols] - want[:, cols])
            bar = 4e-3 * (vmax + np.abs(want[:, cols]))
            assert np.all(err <= bar), (n, h, float(np.max(err - bar)))
            worst = max(worst, float(np.max(err / (vmax + np.abs(want[:, cols])))))
        t0 += n
    return worst


def bf16_values(a):
    return bits_to_f32(f32_to_bf16_bits(a.astype(np.float32)))


LENGTHS = [1, 2, 31, 32, 33, 63, 64, 65, 96, 127, 128, 129, 200, 257, 5]


@pytest.mark.parametrize("d,n_heads", [(32, 4), (64, 3), (128, 2)])
@pytest.mark.parametrize("causal", [False, True])
def test_attention_op_matches_oracle(d, n_heads, causal):
    """Lengths across the 32-query tile, the 32-key tile and the switch to
    four query tiles per block (> 32 tokens), ragged tails, one token."""
    torch = need_gpu()
    say("attention op", d, n_heads, causal)
    rng = np.random.default_rng(d * 10 + n_heads + int(causal))
    T, H = sum(LENGTHS), n_heads * d
    q, k, v = (bf16_values(rng.standard_normal((T, H))) for _ in range(3))
    got = run_case(torch, LENGTHS, n_heads, d, causal, q, k, v)
    say("  worst error / bound scale:", check_against_oracle(got, LENGTHS, n_heads, causal, q, k, v))


@pytest.mark.parametrize("causal", [False, True])
def test_attention_op_growing_scores(causal):
    """Scores that rise along the keys by ~6 (base 2) per key tile, to 58 in
    all: the softmax reference moves up again and again as later key tiles
    arrive (the rescaling path), and most of the weight sits on the last
    visible keys."""
    torch = need_gpu()
    rng = np.random.default_rng(12)
    n_heads, d = 2, 64
    lengths = [257, 100, 40]
    T, H = sum(lengths), n_heads * d
    u = np.where(rng.random((1, H)) < 0.5, -1.0, 1.0)
    q = np.repeat(u, T, axis=0)
    k = np.zeros((T, H))
    t0 = 0
    for n in lengths:
        beta = 5.0 * np.arange(n) / 257.0          # score_j = beta_j * sqrt(d), up to 40
        k[t0:t0 + n] = beta[:, None] * u + 0.05 * rng.standard_normal((n, H))
        t0 += n
    q, k = bf16_values(q), bf16_values(k)
    v = bf16_values(rng.standard_normal((T, H)))
    got = run_case(torch, lengths, n_heads, d, causal, q, k, v)
    check_against_oracle(got, lengths, n_heads, causal, q, k, v)


def test_attention_op_bert_base_shape():
    """Twelve heads of 64 at sequence lengths up to 512 (BERT-base)."""
    torch = need_gpu()
    rng = np.random.default_rng(13)
    lengths = [512, 384, 300, 77, 18, 1]
    n_heads, d = 12, 64
    T, H = sum(lengths), n_heads * d
    q, k, v = (bf16_values(rng.standard_normal((T, H))) for _ in range(3))
    got = run_case(torch, lengths, n_heads, d, False, q, k, v)
    check_against_oracle(got, lengths, n_heads, False, q, k, v)


def test_attention_op_is_deterministic_and_batch_invariant():
    """The same sequence gives bitwise the same context alone and inside a
    batch, and on every run."""
    torch = need_gpu()
    rng = np.random.default_rng(14)
    n_heads, d = 2, 128
    lengths = [70, 33, 150]
    T, H = sum(lengths), n_heads * d
    q, k, v = (bf16_values(rng.standard_normal((T, H))) for _ in range(3))
    a = run_case(torch, lengths, n_heads, d, True, q, k, v)
    b = run_case(torch, lengths, n_heads, d, True, q, k, v)
    assert np.array_equal(a, b)
    s = slice(70, 103)
    alone = run_case(torch, [33], n_heads, d, True, q[s], k[s], v[s])
    assert np.array_equal(alone, a[s])


def test_attention_op_rejects_bad_arguments():
    torch = need_gpu()
    rag = RaggedScores([10, 20], 2, False)
    ok = torch.zeros((30, 3 * 128), dtype=torch.int16, device="cuda")
    ctx = torch.zeros((30, 128), dtype=torch.int16, device="cuda")
    with pytest.raises(EncScoreError):
        attention_fused(rag, ok, ctx, 48)                           # head dim not 32 / 64 / 128
    with pytest.raises(EncScoreError):
        attention_fused(rag, ok, ctx, 128)                          # ld_qkv < 3 * 2 * 128
    narrow = torch.zeros((30, 3 * 128 + 4), dtype=torch.int16, device="cuda")
    with pytest.raises(EncScoreError):
        attention_fused(rag, narrow, ctx, 64)                       # ld_qkv not a multiple of 8
    with pytest.raises(EncScoreError):
        attention_fused(rag, ok[:, :3 * 128].contiguous(), ctx, 64, scale=-1.0)
    rag.close()
