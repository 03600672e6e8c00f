"""Per-kernel parity on the GPU through the C ABI: LayerNorm, ragged Softmax and
the bf16 MFMA GEMM against the oracle's definitions (float64 on the host).

Tolerances: fp32 outputs of the row kernels within 2e-5 (a few ulp of the
O(1) values after fp32 accumulation); bf16 outputs within one bf16 rounding
(2^-8 relative) of the exact value plus the fp32 term; GEMMs within
4e-6 * sum_k |a_k w_k| + bf16 rounding of the output.
"""
import numpy as np
import pytest

import oracle
from encoder_scoring_amd import RaggedScores, gemm_bf16, layernorm, softmax_ragged
from helpers import bf16_bits_to_f32, f32_to_bf16_bits, need_gpu, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("rows,cols", [(1, 128), (37, 312), (1000, 768), (129, 2048), (5, 8192)])
def test_layernorm_op(rows, cols):
    torch = need_gpu()
    say("layernorm", rows, cols)
    rng = np.random.default_rng(rows * 31 + cols)
    x = (rng.standard_normal((rows, cols)) * 0.7 + 0.2).astype(np.float32)
    g = (1 + 0.1 * rng.standard_normal(cols)).astype(np.float32)
    b = (0.1 * rng.standard_normal(cols)).astype(np.float32)
    eps = 1e-5
    dx, dg, db = (torch.from_numpy(a).cuda() for a in (x, g, b))
    y = torch.empty_like(dx)
    ld = cols + 12
    yb = torch.full((rows, ld), 0x1234, dtype=torch.int16, device="cuda")
    layernorm(dx, dg, db, eps, y=y, ybf16=yb)
    torch.cuda.synchronize()
    want = oracle.layer_norm(x.astype(np.float64), g.astype(np.float64), b.astype(np.float64), eps)
    got = y.cpu().numpy()
    assert np.max(np.abs(got - want)) < 2e-5
    bits = yb.cpu().numpy().view(np.uint16)
    assert np.array_equal(bits[:, :cols], f32_to_bf16_bits(got))      # bf16 copy = RNE of fp32
    assert np.all(bits[:, cols:] == 0x1234)                            # padding untouched
    # in place (y aliases x)
    layernorm(dx, dg, db, eps, y=dx)
    torch.cuda.synchronize()
    assert np.array_equal(dx.cpu().numpy(), got)


@pytest.mark.parametrize("rows,cols", [(1, 128), (37, 312), (1000, 768), (5, 8192)])
def test_add_layernorm_op(rows, cols):
    """es_op_add_layernorm = LayerNorm of the float32 sum x + sub: bitwise the
    plain op on that sum (computed by torch in float32), within 2e-5 of the
    float64 oracle on it, and unchanged when y aliases x or sub."""
    torch = need_gpu()
    say("add_layernorm", rows, cols)
    rng = np.random.default_rng(rows * 7 + cols)
    x = (rng.standard_normal((rows, cols)) * 0.7 + 0.2).astype(np.float32)
    u = (rng.standard_normal((rows, cols)) * 1.3 - 0.1).astype(np.float32)
    g = (1 + 0.1 * rng.standard_normal(cols)).astype(np.float32)
    b = (0.1 * rng.standard_normal(cols)).astype(np.float32)
    eps = 1e-5
    dx, du, dg, db = (torch.from_numpy(a).cuda() for a in (x, u, g, b))
    ld = cols + 4
    y, yb = torch.empty_like(dx), torch.full((rows, ld), 0x1234, dtype=torch.int16, device="cuda")
    layernorm(dx, dg, db, eps, y=y, ybf16=yb, sub=du)
    s = dx + du
    y0, yb0 = torch.empty_like(dx), torch.full((rows, ld), 0x1234, dtype=torch.int16, device="cuda")
    layernorm(s, dg, db, eps, y=y0, ybf16=yb0)
    torch.cuda.synchronize()
    assert torch.equal(y, y0) and torch.equal(yb, yb0)
    s64 = x.astype(np.float32) + u.astype(np.float32)        # the float32 sum, as the kernel forms it
    want = oracle.layer_norm(s64.astype(np.float64), g.astype(np.float64), b.astype(np.float64), eps)
    assert np.max(np.abs(y.cpu().numpy() - want)) < 2e-5
    for alias in ("x", "sub"):
        ax, au = dx.clone(), du.clone()
        layernorm(ax, dg, db, eps, y=ax if alias == "x" else au, sub=au)
        torch.cuda.synchronize()
        assert torch.equal(ax if alias == "x" else au, y0), alias
    with pytest.raises(ValueError):
        layernorm(dx, dg, db, eps, y=y, sub=du[:, :-4].contiguous())


def _ragged_rows(lengths, n_heads, causal):
    """(element index of row start, n valid) for every (seq, head, row): rows
    of stride round_up(n, 8), or the causal lower triangle packed with row q
    in round_up(q + 1, 8) elements (summed here row by row)."""
    out = []
    base = 0
    for n in lengths:
        ld = (n + 7) // 8 * 8
        for h in range(n_heads):
            for q in range(n):
                out.append((base, q + 1 if causal else n))
                base += (q + 8) // 8 * 8 if causal else ld
    return out, base


SOFTMAX_LENGTHS = {
    "to560": [1, 2, 7, 8, 9, 16, 17, 31, 32, 33, 63, 64, 65, 100, 127, 128, 129, 255, 256, 257,
              500, 511, 512, 513, 560],
    "to1100": [3, 600, 1024, 1025, 1100],
    "to4096": [5, 4096],
}


@pytest.mark.parametrize("lengths", list(SOFTMAX_LENGTHS), ids=list(SOFTMAX_LENGTHS))
@pytest.mark.parametrize("causal", [0, 1])
def test_softmax_op(causal, lengths):
    torch = need_gpu()
    lengths = SOFTMAX_LENGTHS[lengths]
    A = 3
    say("softmax causal", causal, "lengths up to", max(lengths))
    rag = RaggedScores(lengths, A, causal)
    rows, total = _ragged_rows(lengths, A, causal)
    assert rag.n_elems == total
    rng = np.random.default_rng(11 + causal)
    s = (rng.standard_normal(total) * 3).astype(np.float32)
    ds = torch.from_numpy(s).cuda()
    p32 = torch.full((total,), float("nan"), dtype=torch.float32, device="cuda")
    p16 = torch.full((total,), 0x7FC1, dtype=torch.int16, device="cuda")
    softmax_ragged(rag, ds, p32)
    softmax_ragged(rag, ds, p16)
    torch.cuda.synchronize()
    g32 = p32.cpu().numpy()
    g16 = bf16_bits_to_f32(p16)
    written = np.zeros(total, dtype=bool)
    zeroed = np.zeros(total, dtype=bool)
    worst32 = worst16 = 0.0
    for start, m in rows:
        want = oracle.softmax_rows(s[start:start + m].astype(np.float64)[None])[0]
        worst32 = max(worst32, float(np.max(np.abs(g32[start:start + m] - want))))
        worst16 = max(worst16, float(np.max(np.abs(g16[start:start + m] - want) / (want + 1e-30))))
        written[start:start + m] = True
        zeroed[start + m:start + (m + 7) // 8 * 8] = True     # rest of the row's last 8-chunk
    assert worst32 < 2e-6
    assert worst16 <= 2.0 ** -8 + 1e-5
    assert np.all(g32[zeroed] == 0.0) and np.all(p16.cpu().numpy()[zeroed] == 0)
    untouched = ~(written | zeroed)
    assert np.all(np.isnan(g32[untouched]))                # nothing else written
    assert np.all(p16.cpu().numpy()[untouched] == 0x7FC1)
    # rows sum to one
    assert max(abs(g32[st:st + m].sum() - 1.0) for st, m in rows) < 5e-6
    rag.close()


GEMM_SHAPES = [(1, 64, 64), (37, 936, 320), (300, 768, 768), (1000, 3072, 768),
               (517, 312, 1216), (4100, 2304, 768)]


@pytest.mark.parametrize("M,N,K", GEMM_SHAPES)
@pytest.mark.parametrize("epi", [0, 1, 2, 3])
@pytest.mark.parametrize("tile", [None, 0, 1, 2, 3, 4, 5, 6])
def test_gemm_bf16_op(M, N, K, epi, tile):
    torch = need_gpu()
    say("gemm", M, N, K, "epilogue", epi, "tile", tile)
    rng = np.random.default_rng(M * 7 + N * 3 + K + epi)
    Mr, Nr = -(-M // 256) * 256, -(-N // 256) * 256
    a = f32_to_bf16_bits(rng.standard_normal((Mr, K)).astype(np.float32))
    w = f32_to_bf16_bits((rng.standard_normal((Nr, K)) / np.sqrt(K)).astype(np.float32))
    bias = (0.1 * rng.standard_normal(N)).astype(np.float32)
    ldc = N + 8
    res = (rng.standard_normal((M, ldc))).astype(np.float32)
    a64 = (a.astype(np.uint32) << 16).view(np.float32)[:M].astype(np.float64)
    w64 = (w.astype(np.uint32) << 16).view(np.float32)[:N].astype(np.float64)
    z = a64 @ w64.T + bias
    bound = 4e-6 * (np.abs(a64) @ np.abs(w64).T) + 1e-6
    da = torch.from_numpy(a.view(np.int16)).cuda()
    dw = torch.from_numpy(w.view(np.int16)).cuda()
    db = torch.from_numpy(bias).cuda()
    if epi in (0, 1):
        out = torch.full((M, ldc), 0x5555, dtype=torch.int16, device="cuda")
        gemm_bf16(da, dw, db, out, M, N, K, epi, tile=tile)
        torch.cuda.synchronize()
        got = bf16_bits_to_f32(out)[:, :N].astype(np.float64)
        want = z if epi == 0 else oracle.gelu(z)
        err = np.abs(got - want) - 2.0 ** -8 * np.abs(want)
        assert np.all(err <= bound * (1.0 if epi == 0 else 1.2) + 1e-6)
        assert np.all(out.cpu().numpy()[:, N:] == 0x5555)
    else:
        dres = torch.from_numpy(res).cuda()
        out = torch.full((M, ldc), float("nan"), dtype=torch.float32, device="cuda")
        gemm_bf16(da, dw, db, out, M, N, K, epi, res=dres if epi == 2 else None, tile=tile)
        torch.cuda.synchronize()
        got = out.cpu().numpy()[:, :N].astype(np.float64)
        want = z + res[:, :N] if epi == 2 else z
        assert np.all(np.abs(got - want) <= bound + 1e-6 * np.abs(want))
        assert np.all(np.isnan(out.cpu().numpy()[:, N:]))


@pytest.mark.parametrize("M,N,K", [(300, 768, 768), (4100, 2304, 768), (2100, 3072, 2048),
                                   (700, 2048, 8192)])
def test_gemm_tiles_bitwise_identical(M, N, K):
    """Every tile configuration accumulates each output over K in the same
    order, so all of them give bitwise the same fp32 result (this is what
    makes a sequence's reward independent of the batch it is scored in)."""
    torch = need_gpu()
    say("gemm tiles", M, N, K)
    rng = np.random.default_rng(M + N + K)
    Mr, Nr = -(-M // 256) * 256, -(-N // 256) * 256
    da = torch.from_numpy(f32_to_bf16_bits(rng.standard_normal((Mr, K)).astype(np.float32)).view(np.int16)).cuda()
    dw = torch.from_numpy(f32_to_bf16_bits((rng.standard_normal((Nr, K)) / np.sqrt(K)).astype(np.float32)).view(np.int16)).cuda()
    db = torch.from_numpy((0.1 * rng.standard_normal(N)).astype(np.float32)).cuda()
    outs = []
    for tile in (0, 1, 2, 3, 4, 5, 6):
        out = torch.empty((M, N), dtype=torch.float32, device="cuda")
        gemm_bf16(da, dw, db, out, M, N, K, 3, tile=tile)
        outs.append(out)
    torch.cuda.synchronize()
    assert all(torch.equal(outs[0], o) for o in outs[1:])


def test_gemm_rejects_bad_shapes():
    torch = need_gpu()
    from encoder_scoring_amd import EncScoreError
    a = torch.zeros((256, 96), dtype=torch.int16, device="cuda")
    w = torch.zeros((256, 96), dtype=torch.int16, device="cuda")
    bias = torch.zeros(64, dtype=torch.float32, device="cuda")
    out = torch.zeros((4, 64), dtype=torch.int16, device="cuda")
    with pytest.raises(EncScoreError):
        gemm_bf16(a, w, bias, out, 4, 64, 96, 0)      # K not a multiple of 64
    a64 = torch.zeros((256, 64), dtype=torch.int16, device="cuda")
    w64 = torch.zeros((256, 64), dtype=torch.int16, device="cuda")
    with pytest.raises(EncScoreError):
        gemm_bf16(a64, w64, bias, out, 4, 64, 64, 0, tile=7)  # no such tile


def test_bf16_conversion_ties_and_specials():
    """The bf16 epilogue's float -> bf16 conversion rounds to nearest, ties to
    even: with zero operands every output is exactly bf16(bias[n]), and the
    biases are exact midpoints between neighbouring bf16 values (even and odd
    lower neighbour), infinities, subnormals, and the largest finite values."""
    torch = need_gpu()
    rng = np.random.default_rng(11)
    hi = rng.integers(0x0080, 0x7F00, size=96).astype(np.uint32)       # bf16 patterns
    mids = ((hi << 16) | 0x8000).view(np.float32)                       # exact ties
    mids = np.concatenate([mids, -mids[:32]])
    specials = np.array([np.inf, -np.inf, 0.0, -0.0, 1e-40, -3e-39, 3.3895314e38, -3.3895314e38,
                         1.0 + 2 ** -9, 1.0 + 3 * 2 ** -9, 2 ** -126, 0.1], dtype=np.float32)
    bias = np.concatenate([mids, specials]).astype(np.float32)
    N = bias.size
    M, K = 33, 64
    a = torch.zeros((256, K), dtype=torch.int16, device="cuda")
    w = torch.zeros((-(-N // 256) * 256, K), dtype=torch.int16, device="cuda")
    out = torch.zeros((M, N + (-N) % 4), dtype=torch.int16, device="cuda")
    gemm_bf16(a, w, torch.from_numpy(bias).cuda(), out, M, N, K, 0)
    torch.cuda.synchronize()
    got = out.cpu().numpy().view(np.uint16)[:, :N]
    want = f32_to_bf16_bits((np.float32(0.0) + bias).astype(np.float32))   # acc (+0) + bias
    assert np.array_equal(got, np.broadcast_to(want, got.shape))
    # NaN stays NaN
    nan_bias = torch.full((4,), float("nan"), device="cuda")
    out4 = torch.zeros((M, 4), dtype=torch.int16, device="cuda")
    gemm_bf16(a, torch.zeros((256, K), dtype=torch.int16, device="cuda"), nan_bias, out4, M, 4, K, 0)
    torch.cuda.synchronize()
    assert np.all(np.isnan(bf16_bits_to_f32(out4)))
