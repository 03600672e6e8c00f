"""The last-token refinement's kernels on caller buffers, against float64
references written out from their definitions.

Split-operand layout (es_op_split): each fp32 activation a as hi = bf16(a),
lo = bf16(a - hi), both rounded to nearest even; checked bit for bit, and
|a - hi - lo| <= 2^-16 |a| (each rounding keeps 8 significant bits).  GEMM
(es_op_gemm_split): A W^T + bias (+ residual, or GELU) with A given as
hi + lo; per product the split leaves at most 2^-16 |a w|, so the error is
tested against 2^-14 sqrt(sum_k (a_k w_k)^2) (random rounding errors add
like a random walk) plus 2^-22 sum_k |a_k w_k| for the fp32 accumulation.
A GEMM that used hi alone (bf16 rounding, 2^-8 per product) exceeds that
bound about 100-fold at its worst output (numpy, K = 64 .. 8192; hi + lo
stays at 0.13 - 0.17 of it).  The LayerNorm and the last-query attention (fp32
arithmetic, outputs split: 2^-16 relative, plus a few 1e-6 of the output
scale for the fp32 sums) against float64.  Shapes cover one to five row
tiles, ragged row and column tails, and K over 1, 2 and 4 wavefronts.
"""
import math

import numpy as np
import pytest

import oracle
from encoder_scoring_amd import EncScoreError, RaggedScores, attention_last, gemm_split, layernorm_split, split_rows
from helpers import bits_to_f64, f32_to_bf16_bits, need_gpu, say, split_decode

pytestmark = pytest.mark.gpu


def _m32(M):
    return -(-M // 32) * 32


def _split_of(torch, a):
    """fp32 numpy [M, K] -> device split-operand buffer (through es_op_split)."""
    M, K = a.shape
    out = torch.zeros(2 * _m32(M) * K, dtype=torch.int16, device="cuda")
    split_rows(torch.from_numpy(np.ascontiguousarray(a)).cuda(), out)
    return out


def _decoded(out, M, K):
    hi, lo = split_decode(out.cpu().numpy(), M, K)
    return bits_to_f64(hi)[:M] + bits_to_f64(lo)[:M]


@pytest.mark.parametrize("M,K", [(1, 16), (33, 64), (77, 320), (155, 2048)])
def test_split_is_two_roundings(M, K):
    torch = need_gpu()
    rng = np.random.default_rng(M * 31 + K)
    a = (rng.standard_normal((M, K)) * np.exp2(rng.integers(-20, 21, (M, K)))).astype(np.float32)
    out = torch.full((2 * _m32(M) * K,), 0x5555, dtype=torch.int16, device="cuda")
    split_rows(torch.from_numpy(a).cuda(), out)
    hi, lo = split_decode(out.cpu().numpy(), M, K)
    want_hi = f32_to_bf16_bits(a)
    rest = a - (want_hi.astype(np.uint32) << 16).view(np.float32)  # exact in float32
    assert np.array_equal(hi[:M], want_hi)
    assert np.array_equal(lo[:M], f32_to_bf16_bits(rest))
    assert np.all(hi[M:] == 0) and np.all(lo[M:] == 0)
    a64 = a.astype(np.float64)
    assert np.all(np.abs(a64 - bits_to_f64(hi[:M]) - bits_to_f64(lo[:M])) <= 2.0 ** -16 * np.abs(a64))


SHAPES = [(1, 32, 64), (31, 96, 128), (33, 2048, 256), (77, 96, 320), (155, 6144, 2048),
          (155, 2048, 8192), (200, 1024, 512)]


@pytest.mark.parametrize("M,N,K", SHAPES)
@pytest.mark.parametrize("epi", [1, 2, 3])
def test_gemm_split(M, N, K, epi):
    torch = need_gpu()
    say("gemm_split", M, N, K, "epilogue", epi)
    rng = np.random.default_rng(M * 7 + N * 3 + K + epi)
    a = rng.standard_normal((M, K)).astype(np.float32)
    w = f32_to_bf16_bits((rng.standard_normal((N, K)) / np.sqrt(K)).astype(np.float32))
    bias = (0.1 * rng.standard_normal(N)).astype(np.float32)
    a64 = a.astype(np.float64)
    w64 = bits_to_f64(w)
    z = a64 @ w64.T + bias
    rss = np.sqrt((a64 ** 2) @ (w64 ** 2).T)
    scale = 2.0 ** -14 * rss + 2.0 ** -22 * (np.abs(a64) @ np.abs(w64).T + np.abs(bias))
    da = _split_of(torch, a)
    dw = torch.from_numpy(w.view(np.int16)).cuda()
    db = torch.from_numpy(bias).cuda()
    if epi == 1:
        out = torch.zeros(2 * _m32(M) * N, dtype=torch.int16, device="cuda")
        gemm_split(da, dw, db, M, N, K, 1, out_split=out)
        torch.cuda.synchronize()
        got = _decoded(out, M, N)
        want = oracle.gelu(z)
        err = np.abs(got - want)
        bound = 1.2 * scale + 2.0 ** -16 * np.abs(want) + 1e-7  # GELU' <= 1.13; the output's split
    else:
        ldc = N + 4
        res = rng.standard_normal((M, ldc)).astype(np.float32)
        out = torch.from_numpy(np.full((M, ldc), np.nan, dtype=np.float32)).cuda()
        dres = torch.from_numpy(res).cuda() if epi == 2 else None
        gemm_split(da, dw, db, M, N, K, epi, out=out, res=dres)
        torch.cuda.synchronize()
        o = out.cpu().numpy()
        assert np.all(np.isnan(o[:, N:]))
        got = o[:, :N].astype(np.float64)
        want = z + res[:, :N] if epi == 2 else z
        err = np.abs(got - want)
        bound = scale + 2.0 ** -23 * np.abs(want)
    worst = float(np.max(err / bound))
    say(f"  max err {err.max():.3e}, worst err / bound {worst:.3f}")
    assert worst <= 1.0


def test_gemm_split_residual_in_place():
    """res may be the output (the refinement adds into its residual rows)."""
    torch = need_gpu()
    rng = np.random.default_rng(5)
    M, N, K = 45, 256, 512
    a = rng.standard_normal((M, K)).astype(np.float32)
    w = f32_to_bf16_bits((rng.standard_normal((N, K)) / np.sqrt(K)).astype(np.float32))
    bias = (0.1 * rng.standard_normal(N)).astype(np.float32)
    x = rng.standard_normal((M, N)).astype(np.float32)
    da, dw, db = _split_of(torch, a), torch.from_numpy(w.view(np.int16)).cuda(), torch.from_numpy(bias).cuda()
    sep = torch.empty((M, N), dtype=torch.float32, device="cuda")
    dx = torch.from_numpy(x).cuda()
    gemm_split(da, dw, db, M, N, K, 2, out=sep, res=dx)
    gemm_split(da, dw, db, M, N, K, 2, out=dx, res=dx)
    torch.cuda.synchronize()
    assert torch.equal(sep, dx)


@pytest.mark.parametrize("rows,cols", [(1, 64), (37, 768), (155, 2048)])
def test_layernorm_split(rows, cols):
    torch = need_gpu()
    rng = np.random.default_rng(rows + cols)
    x = (3.0 * rng.standard_normal((rows, cols)) + 1.0).astype(np.float32)
    g = (1.0 + 0.1 * rng.standard_normal(cols)).astype(np.float32)
    b = (0.1 * rng.standard_normal(cols)).astype(np.float32)
    out = torch.zeros(2 * _m32(rows) * cols, dtype=torch.int16, device="cuda")
    layernorm_split(torch.from_numpy(x).cuda(), torch.from_numpy(g).cuda(), torch.from_numpy(b).cuda(),
                    1e-5, out)
    torch.cuda.synchronize()
    got = _decoded(out, rows, cols)
    want = oracle.layer_norm(x.astype(np.float64), g.astype(np.float64), b.astype(np.float64), 1e-5)
    err = np.abs(got - want)
    say(f"layernorm_split {rows}x{cols}: max err {err.max():.3e}")
    assert np.all(err <= 2.0 ** -16 * np.abs(want) + 4e-6)


@pytest.mark.parametrize("head_dim", [32, 64, 128])
@pytest.mark.parametrize("lengths", [[1, 5, 40], [300, 77, 1, 1024]])
def test_attention_last(head_dim, lengths):
    torch = need_gpu()
    A = 3
    width = A * head_dim
    kc = -(-width // 64) * 64 + 64  # a zero band after the heads
    rng = np.random.default_rng(head_dim + sum(lengths))
    T, n = int(sum(lengths)), len(lengths)
    qkv = f32_to_bf16_bits(rng.standard_normal((T, 3 * width + 8)).astype(np.float32))
    ql = rng.standard_normal((n, 3 * width)).astype(np.float32)
    rag = RaggedScores(np.asarray(lengths, dtype=np.int32), A, 1)
    out = torch.full((2 * _m32(n) * kc,), 0x5555, dtype=torch.int16, device="cuda")
    attention_last(rag, torch.from_numpy(qkv.view(np.int16)).cuda(), torch.from_numpy(ql).cuda(), out,
                   head_dim, kc)
    torch.cuda.synchronize()
    rag.close()
    got = _decoded(out, n, kc)
    scale = 1.0 / math.sqrt(head_dim)
    q64 = bits_to_f64(qkv)
    t0 = 0
    for i, L in enumerate(lengths):
        rows = q64[t0:t0 + L]
        for h in range(A):
            sl = slice(h * head_dim, (h + 1) * head_dim)
            K = rows[:, width:2 * width][:, sl].copy()
            V = rows[:, 2 * width:3 * width][:, sl].copy()
            K[-1] = ql[i, width:2 * width][sl]
            V[-1] = ql[i, 2 * width:][sl]
            s = scale * (K @ ql[i, :width][sl].astype(np.float64))
            p = oracle.softmax_rows(s[None])[0]
            want = p @ V
            err = np.abs(got[i, sl] - want)
            assert np.all(err <= 2.0 ** -16 * np.abs(want) + 1e-5 * np.abs(V).max()), (i, h, err.max())
        t0 += L
    assert np.all(got[:, width:] == 0.0)


def test_attention_last_refuses_longer_sequences():
    torch = need_gpu()
    rag = RaggedScores(np.array([3, 1025], dtype=np.int32), 2, 1)
    qkv = torch.zeros((1028, 3 * 64), dtype=torch.int16, device="cuda")
    ql = torch.zeros((2, 3 * 64), dtype=torch.float32, device="cuda")
    out = torch.zeros(2 * 32 * 64, dtype=torch.int16, device="cuda")
    with pytest.raises(EncScoreError, match="ES_ERR_RANGE"):
        attention_last(rag, qkv, ql, out, 32, 64)
    rag.close()
