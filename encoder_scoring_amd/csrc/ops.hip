// Single-kernel entry points: the LayerNorm, Softmax and GEMM kernels of the
// hot path on caller buffers, for per-kernel parity tests and measurement.
#include <cinttypes>
#include <vector>

#include "common.h"
#include "kernels.h"

using es::fail;

#define HIP_TRY(expr)                                                                     \
  do {                                                                                    \
    hipError_t _e = (expr);                                                               \
    if (_e != hipSuccess)                                                                 \
      return fail(ES_ERR_HIP, "%s failed: %s", #expr, hipGetErrorString(_e));             \
  } while (0)

struct es_ragged {
  void *dev = nullptr;  // off | sbase | items
  es::Ragged r;
  int n_heads = 0, causal = 0;
};

extern "C" es_status es_op_layernorm(const float *d_x, const float *d_gamma, const float *d_beta,
                                     int64_t rows, int32_t cols, float eps, float *d_y,
                                     uint16_t *d_ybf16, int32_t ld_bf16, void *stream) {
  if (!d_x || !d_gamma || !d_beta || (!d_y && !d_ybf16))
    return fail(ES_ERR_ARG, "es_op_layernorm: NULL pointer");
  if (rows < 0 || cols < 4 || cols % 4 || cols > 8192 || (d_ybf16 && (ld_bf16 < cols || ld_bf16 % 4)))
    return fail(ES_ERR_ARG, "es_op_layernorm: rows=%" PRId64 " cols=%d ld_bf16=%d", rows, cols, ld_bf16);
  HIP_TRY(es::launch_layernorm(true, d_x, nullptr, d_gamma, d_beta, rows, cols, eps, d_y, d_ybf16,
                               ld_bf16, cols, static_cast<hipStream_t>(stream)));
  return ES_OK;
}

extern "C" es_status es_op_add_layernorm(const float *d_x, const float *d_sub, const float *d_gamma,
                                         const float *d_beta, int64_t rows, int32_t cols, float eps,
                                         float *d_y, uint16_t *d_ybf16, int32_t ld_bf16,
                                         void *stream) {
  if (!d_x || !d_sub || !d_gamma || !d_beta || (!d_y && !d_ybf16))
    return fail(ES_ERR_ARG, "es_op_add_layernorm: NULL pointer");
  if (rows < 0 || cols < 4 || cols % 4 || cols > 8192 || (d_ybf16 && (ld_bf16 < cols || ld_bf16 % 4)))
    return fail(ES_ERR_ARG, "es_op_add_layernorm: rows=%" PRId64 " cols=%d ld_bf16=%d", rows, cols,
                ld_bf16);
  HIP_TRY(es::launch_layernorm(true, d_x, d_sub, d_gamma, d_beta, rows, cols, eps, d_y, d_ybf16,
                               ld_bf16, cols, static_cast<hipStream_t>(stream)));
  return ES_OK;
}

extern "C" es_status es_ragged_create(const int32_t *h_lengths, int32_t n_seqs, int32_t n_heads,
                                      int32_t causal, es_ragged **out, int64_t *n_elems) {
  if (!h_lengths || !out || n_seqs < 1 || n_heads < 1 || (causal != 0 && causal != 1))
    return fail(ES_ERR_ARG, "es_ragged_create: bad arguments");
  *out = nullptr;
  std::vector<int32_t> off(n_seqs + 1, 0);
  std::vector<int64_t> sbase(n_seqs);
  std::vector<int32_t> items, sm_items, sm_wide, fitems, mitems;
  int64_t acc = 0;
  int max_len = 0;
  for (int32_t i = 0; i < n_seqs; ++i) {
    const int n = h_lengths[i];
    if (n < 1 || n > 4096) return fail(ES_ERR_RANGE, "es_ragged_create: length %d outside [1, 4096]", n);
    if ((int64_t)off[i] + n > INT32_MAX) return fail(ES_ERR_RANGE, "es_ragged_create: too many tokens");
    off[i + 1] = off[i] + n;
    sbase[i] = acc;
    acc += (int64_t)n_heads * es::score_block(n, causal != 0);
    max_len = max_len > n ? max_len : n;
    for (int q0 = 0; q0 < n; q0 += es::kQTile) {
      items.push_back(i);
      items.push_back(q0);
    }
    // fused attention work, split by length as in a scoring pass
    auto &fl = n > es::kMwMinLen ? mitems : fitems;
    for (int q0 = 0; q0 < n; q0 += n > es::kMwMinLen ? 4 * es::kQTile : es::kQTile) {
      fl.push_back(i);
      fl.push_back(q0);
    }
    es::softmax_items(n, n_heads, causal != 0, [&](int r0, bool wide) {
      auto &dst = wide ? sm_wide : sm_items;
      dst.push_back(i);
      dst.push_back(r0);
    });
  }
  const int32_t n_sm_narrow = (int32_t)(sm_items.size() / 2);
  sm_items.insert(sm_items.end(), sm_wide.begin(), sm_wide.end());
  const size_t b_off = es::round_up((int64_t)off.size() * 4, 16);
  const size_t b_sb = es::round_up((int64_t)sbase.size() * 8, 16);
  const size_t b_it = es::round_up((int64_t)items.size() * 4, 16);
  const size_t b_sm = es::round_up((int64_t)sm_items.size() * 4, 16);
  const size_t b_fi = es::round_up((int64_t)fitems.size() * 4, 16);
  const size_t bytes = b_off + b_sb + b_it + b_sm + b_fi + mitems.size() * 4 + 16;
  es_ragged *g = new es_ragged();
  hipError_t e = hipMalloc(&g->dev, bytes);
  if (e == hipSuccess) e = hipMemcpy(g->dev, off.data(), off.size() * 4, hipMemcpyHostToDevice);
  if (e == hipSuccess)
    e = hipMemcpy((char *)g->dev + b_off, sbase.data(), sbase.size() * 8, hipMemcpyHostToDevice);
  if (e == hipSuccess)
    e = hipMemcpy((char *)g->dev + b_off + b_sb, items.data(), items.size() * 4, hipMemcpyHostToDevice);
  if (e == hipSuccess)
    e = hipMemcpy((char *)g->dev + b_off + b_sb + b_it, sm_items.data(), sm_items.size() * 4,
                  hipMemcpyHostToDevice);
  if (e == hipSuccess && !fitems.empty())
    e = hipMemcpy((char *)g->dev + b_off + b_sb + b_it + b_sm, fitems.data(), fitems.size() * 4,
                  hipMemcpyHostToDevice);
  if (e == hipSuccess && !mitems.empty())
    e = hipMemcpy((char *)g->dev + b_off + b_sb + b_it + b_sm + b_fi, mitems.data(),
                  mitems.size() * 4, hipMemcpyHostToDevice);
  if (e != hipSuccess) {
    if (g->dev) (void)hipFree(g->dev);
    delete g;
    return fail(ES_ERR_HIP, "es_ragged_create: %s", hipGetErrorString(e));
  }
  g->r.off = (const int32_t *)g->dev;
  g->r.sbase = (const int64_t *)((char *)g->dev + b_off);
  g->r.items = (const int32_t *)((char *)g->dev + b_off + b_sb);
  g->r.n_seqs = n_seqs;
  g->r.n_items = (int32_t)(items.size() / 2);
  g->r.sm_items = (const int32_t *)((char *)g->dev + b_off + b_sb + b_it);
  g->r.n_sm_items = (int32_t)(sm_items.size() / 2);
  g->r.n_sm_narrow = n_sm_narrow;
  g->r.fused_items = (const int32_t *)((char *)g->dev + b_off + b_sb + b_it + b_sm);
  g->r.n_fused_items = (int32_t)(fitems.size() / 2);
  g->r.mw_items = (const int32_t *)((char *)g->dev + b_off + b_sb + b_it + b_sm + b_fi);
  g->r.n_mw_items = (int32_t)(mitems.size() / 2);
  g->r.max_len = max_len;
  g->r.n_tokens = off[n_seqs];
  g->n_heads = n_heads;
  g->causal = causal;
  if (n_elems) *n_elems = acc;
  *out = g;
  return ES_OK;
}

extern "C" void es_ragged_free(es_ragged *r) {
  if (!r) return;
  (void)hipDeviceSynchronize();
  (void)hipFree(r->dev);
  delete r;
}

extern "C" es_status es_op_softmax(const es_ragged *r, const float *d_scores, void *d_p,
                                   int32_t p_bf16, void *stream) {
  if (!r || !d_scores || !d_p) return fail(ES_ERR_ARG, "es_op_softmax: NULL pointer");
  HIP_TRY(es::launch_softmax(p_bf16 != 0, d_scores, d_p, r->r, r->n_heads, r->causal != 0,
                             static_cast<hipStream_t>(stream)));
  return ES_OK;
}

extern "C" es_status es_op_attention(const es_ragged *r, const uint16_t *d_qkv, int32_t ld_qkv,
                                     int32_t head_dim, float scale, uint16_t *d_ctx, int32_t ld_ctx,
                                     void *stream) {
  if (!r || !d_qkv || !d_ctx) return fail(ES_ERR_ARG, "es_op_attention: NULL pointer");
  const int64_t width = (int64_t)r->n_heads * head_dim;
  if ((head_dim != 32 && head_dim != 64 && head_dim != 128) || ld_qkv < 3 * width || ld_qkv % 8 ||
      ld_ctx < width || ld_ctx % 4 || !(scale > 0.f))
    return fail(ES_ERR_ARG, "es_op_attention: head_dim=%d ld_qkv=%d ld_ctx=%d scale=%g (n_heads=%d)",
                head_dim, ld_qkv, ld_ctx, (double)scale, r->n_heads);
  HIP_TRY(es::launch_attn_fused(d_qkv, ld_qkv, r->n_heads, head_dim, scale, r->causal != 0, r->r,
                                d_ctx, ld_ctx, static_cast<hipStream_t>(stream)));
  return ES_OK;
}

static es_status gemm_bf16_checked(const char *who, const uint16_t *d_a, int32_t lda,
                                   const uint16_t *d_w, const float *d_bias, const float *d_res,
                                   void *d_out, int32_t ldc, int32_t M, int32_t N, int32_t K,
                                   int32_t epilogue, int32_t tile, void *stream) {
  if (!d_a || !d_w || !d_bias || !d_out || (epilogue == es::kEpiResidual && !d_res))
    return fail(ES_ERR_ARG, "%s: NULL pointer", who);
  if (M < 0 || N < 0 || K <= 0 || K % 64 || lda < K || lda % 8 || ldc < N || ldc % 4 || epilogue < 0 ||
      epilogue > 3)
    return fail(ES_ERR_ARG, "%s: M=%d N=%d K=%d lda=%d ldc=%d epilogue=%d", who, M, N, K, lda, ldc,
                epilogue);
  if (tile < -1 || tile >= es::kGemmTiles) return fail(ES_ERR_ARG, "%s: tile %d", who, tile);
  const hipStream_t st = static_cast<hipStream_t>(stream);
  if (tile < 0) {
    HIP_TRY(es::launch_gemm_bf16(d_a, lda, d_w, d_bias, d_res, d_out, ldc, M, N, K, epilogue, st));
  } else {
    HIP_TRY(es::launch_gemm_bf16_tile(tile, d_a, lda, d_w, d_bias, d_res, d_out, ldc, M, N, K,
                                      epilogue, st));
  }
  return ES_OK;
}

extern "C" es_status es_op_gemm_bf16(const uint16_t *d_a, int32_t lda, const uint16_t *d_w,
                                     const float *d_bias, const float *d_res, void *d_out,
                                     int32_t ldc, int32_t M, int32_t N, int32_t K, int32_t epilogue,
                                     void *stream) {
  return gemm_bf16_checked("es_op_gemm_bf16", d_a, lda, d_w, d_bias, d_res, d_out, ldc, M, N, K,
                           epilogue, -1, stream);
}

extern "C" es_status es_op_gemm_bf16_tile(const uint16_t *d_a, int32_t lda, const uint16_t *d_w,
                                          const float *d_bias, const float *d_res, void *d_out,
                                          int32_t ldc, int32_t M, int32_t N, int32_t K,
                                          int32_t epilogue, int32_t tile, void *stream) {
  return gemm_bf16_checked("es_op_gemm_bf16_tile", d_a, lda, d_w, d_bias, d_res, d_out, ldc, M, N,
                           K, epilogue, tile, stream);
}

// ---- the refinement's split-operand kernels (last-token rows in fp32)

extern "C" es_status es_op_split(const float *d_a, int32_t lda, int32_t M, int32_t K,
                                 uint16_t *d_out, void *stream) {
  if (!d_a || !d_out) return fail(ES_ERR_ARG, "es_op_split: NULL pointer");
  if (M < 0 || K <= 0 || K % 16 || lda < K || lda % 4)
    return fail(ES_ERR_ARG, "es_op_split: M=%d K=%d lda=%d", M, K, lda);
  HIP_TRY(es::launch_split_rows(d_a, lda, M, K, d_out, static_cast<hipStream_t>(stream)));
  return ES_OK;
}

extern "C" es_status es_op_layernorm_split(const float *d_x, const float *d_gamma,
                                           const float *d_beta, int32_t rows, int32_t cols,
                                           float eps, uint16_t *d_out, void *stream) {
  if (!d_x || !d_gamma || !d_beta || !d_out) return fail(ES_ERR_ARG, "es_op_layernorm_split: NULL pointer");
  if (rows < 0 || cols <= 0 || cols % 16) return fail(ES_ERR_ARG, "es_op_layernorm_split: rows=%d cols=%d", rows, cols);
  HIP_TRY(es::launch_layernorm_split(d_x, d_gamma, d_beta, rows, cols, eps, d_out,
                                     static_cast<hipStream_t>(stream)));
  return ES_OK;
}

extern "C" es_status es_op_gemm_split(const uint16_t *d_a, const uint16_t *d_w, const float *d_bias,
                                      const float *d_res, float *d_out, uint16_t *d_out_split,
                                      int32_t ldc, int32_t M, int32_t N, int32_t K, int32_t epilogue,
                                      void *stream) {
  if (!d_a || !d_w || !d_bias) return fail(ES_ERR_ARG, "es_op_gemm_split: NULL pointer");
  if (epilogue != es::kEpiGelu && epilogue != es::kEpiResidual && epilogue != es::kEpiF32)
    return fail(ES_ERR_ARG, "es_op_gemm_split: epilogue %d", epilogue);
  if (epilogue == es::kEpiGelu ? !d_out_split : (!d_out || (epilogue == es::kEpiResidual && !d_res)))
    return fail(ES_ERR_ARG, "es_op_gemm_split: NULL output or residual");
  if (M < 0 || N <= 0 || K <= 0 || K % 64 || (epilogue == es::kEpiGelu ? N % 16 != 0 : ldc < N))
    return fail(ES_ERR_ARG, "es_op_gemm_split: M=%d N=%d K=%d ldc=%d", M, N, K, ldc);
  HIP_TRY(es::launch_gemm_split(d_a, d_w, d_bias, d_res, d_out, d_out_split, ldc, M, N, K, epilogue,
                                static_cast<hipStream_t>(stream)));
  return ES_OK;
}

extern "C" es_status es_op_attention_last(const es_ragged *r, const uint16_t *d_qkv, int32_t ld_qkv,
                                          const float *d_ql, int32_t ld_ql, int32_t head_dim,
                                          float scale, uint16_t *d_ctx_split, int32_t kc,
                                          void *stream) {
  if (!r || !d_qkv || !d_ql || !d_ctx_split) return fail(ES_ERR_ARG, "es_op_attention_last: NULL pointer");
  const int64_t width = (int64_t)r->n_heads * head_dim;
  if ((head_dim != 32 && head_dim != 64 && head_dim != 128) || ld_qkv < 3 * width || ld_qkv % 8 ||
      ld_ql < 3 * width || kc < width || kc % 16 || !(scale > 0.f))
    return fail(ES_ERR_ARG, "es_op_attention_last: head_dim=%d ld_qkv=%d ld_ql=%d kc=%d scale=%g (n_heads=%d)",
                head_dim, ld_qkv, ld_ql, kc, (double)scale, r->n_heads);
  if (r->r.max_len > es::kLastMaxKeysHost)
    return fail(ES_ERR_RANGE, "es_op_attention_last: a sequence of %d tokens (at most %d)", r->r.max_len,
                es::kLastMaxKeysHost);
  HIP_TRY(es::launch_attn_last(d_qkv, ld_qkv, d_ql, ld_ql, r->n_heads, head_dim, scale, r->r,
                               d_ctx_split, kc, static_cast<hipStream_t>(stream)));
  return ES_OK;
}
