// Weight blob parsing (host only; no HIP calls).
#include "blob.h"

#include <cinttypes>
#include <cmath>
#include <cstring>

namespace es {

namespace {

struct Cursor {
  const uint8_t *base;
  int64_t size, pos;
  bool take(TensorView *t, int64_t rows, int64_t cols, int elem) {
    const int64_t bytes = rows * cols * elem;
    if (pos + bytes > size) return false;
    t->data = base + pos;
    t->rows = rows;
    t->cols = cols;
    t->elem = elem;
    pos += bytes;
    return true;
  }
};

}  // namespace

es_status parse_blob(const void *p, int64_t nbytes, ParsedBlob *out) {
  if (!p || nbytes < (int64_t)sizeof(BlobHeader))
    return fail(ES_ERR_FORMAT, "blob: %" PRId64 " bytes is shorter than the 64-byte header", nbytes);
  BlobHeader h;
  std::memcpy(&h, p, sizeof(h));
  if (std::memcmp(h.magic, "ESW1", 4) != 0) return fail(ES_ERR_FORMAT, "blob: bad magic");
  if (h.version != 1) return fail(ES_ERR_FORMAT, "blob: unsupported version %u", h.version);
  if (h.n_layers < 1 || h.n_layers > 256) return fail(ES_ERR_FORMAT, "blob: n_layers=%u", h.n_layers);
  if (h.hidden < 4 || h.hidden > (uint32_t)kMaxHidden || h.hidden % 4)
    return fail(ES_ERR_FORMAT, "blob: hidden=%u (need a multiple of 4, <= %d)", h.hidden, kMaxHidden);
  if (h.n_heads < 1 || h.hidden % h.n_heads)
    return fail(ES_ERR_FORMAT, "blob: n_heads=%u does not divide hidden=%u", h.n_heads, h.hidden);
  if (h.hidden / h.n_heads > (uint32_t)kMaxHeadDim)
    return fail(ES_ERR_FORMAT, "blob: head_dim=%u above %d", h.hidden / h.n_heads, kMaxHeadDim);
  if (h.ffn < 1 || h.ffn > 65536) return fail(ES_ERR_FORMAT, "blob: ffn=%u", h.ffn);
  if (h.vocab < 1 || h.vocab > (1u << 24)) return fail(ES_ERR_FORMAT, "blob: vocab=%u", h.vocab);
  if (h.max_pos < 1 || h.max_pos > (uint32_t)kMaxPos)
    return fail(ES_ERR_FORMAT, "blob: max_pos=%u (limit %d)", h.max_pos, kMaxPos);
  if (h.pre_ln > 1 || h.causal > 1) return fail(ES_ERR_FORMAT, "blob: bad pre_ln/causal flag");
  if (h.act != 0) return fail(ES_ERR_FORMAT, "blob: unknown activation %u", h.act);
  if (h.wdtype > 1) return fail(ES_ERR_FORMAT, "blob: unknown weight dtype %u", h.wdtype);
  if (!(h.eps >= 0.0f) || !std::isfinite(h.eps) || !std::isfinite(h.reward_offset))
    return fail(ES_ERR_FORMAT, "blob: eps / reward_offset not finite");

  const int64_t H = h.hidden, F = h.ffn, V = h.vocab, P = h.max_pos;
  const int me = h.wdtype == 1 ? 2 : 4;  // matrix element size
  Cursor c{static_cast<const uint8_t *>(p), nbytes, (int64_t)sizeof(BlobHeader)};
  bool ok = c.take(&out->tok_emb, V, H, me) && c.take(&out->pos_emb, P, H, me) &&
            c.take(&out->norm_g, 1, H, 4) && c.take(&out->norm_b, 1, H, 4);
  out->layers.assign(h.n_layers, LayerViews{});
  for (uint32_t l = 0; ok && l < h.n_layers; ++l) {
    LayerViews &L = out->layers[l];
    ok = c.take(&L.w_qkv, 3 * H, H, me) && c.take(&L.b_qkv, 1, 3 * H, 4) &&
         c.take(&L.w_o, H, H, me) && c.take(&L.b_o, 1, H, 4) && c.take(&L.ln1_g, 1, H, 4) &&
         c.take(&L.ln1_b, 1, H, 4) && c.take(&L.w_1, F, H, me) && c.take(&L.b_1, 1, F, 4) &&
         c.take(&L.w_2, H, F, me) && c.take(&L.b_2, 1, H, 4) && c.take(&L.ln2_g, 1, H, 4) &&
         c.take(&L.ln2_b, 1, H, 4);
  }
  ok = ok && c.take(&out->head_w, 1, H, 4) && c.take(&out->head_b, 1, 1, 4);
  if (!ok) return fail(ES_ERR_FORMAT, "blob: truncated (%" PRId64 " bytes)", nbytes);
  if (c.pos != nbytes)
    return fail(ES_ERR_FORMAT, "blob: %" PRId64 " trailing bytes", nbytes - c.pos);
  out->h = h;
  return ES_OK;
}

}  // namespace es

// Host only: validate a blob and report the model it holds.
extern "C" es_status es_blob_info(const void *h_blob, int64_t nbytes, es_model_info_t *info) {
  if (!h_blob || !info) return es::fail(ES_ERR_ARG, "es_blob_info: NULL argument");
  es::ParsedBlob pb;
  const es_status s = es::parse_blob(h_blob, nbytes, &pb);
  if (s != ES_OK) return s;
  std::memset(info, 0, sizeof(*info));
  info->n_layers = (int32_t)pb.h.n_layers;
  info->hidden = (int32_t)pb.h.hidden;
  info->n_heads = (int32_t)pb.h.n_heads;
  info->head_dim = (int32_t)(pb.h.hidden / pb.h.n_heads);
  info->ffn = (int32_t)pb.h.ffn;
  info->vocab = (int32_t)pb.h.vocab;
  info->max_pos = (int32_t)pb.h.max_pos;
  info->pre_ln = (int32_t)pb.h.pre_ln;
  info->causal = (int32_t)pb.h.causal;
  info->bf16 = pb.h.wdtype == 1;
  info->eps = pb.h.eps;
  info->reward_offset = pb.h.reward_offset;
  es::clear_error();
  return ES_OK;
}
