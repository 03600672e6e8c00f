// Weight blob ("ESW1") parsing: header validation and tensor views into the
// caller's bytes.  Host only.
#pragma once

#include <cstdint>
#include <vector>

#include "common.h"

namespace es {

struct BlobHeader {
  char magic[4];
  uint32_t version;
  uint32_t n_layers, hidden, n_heads, ffn, vocab, max_pos;
  uint32_t pre_ln, causal, act, wdtype;
  float eps, reward_offset;
  uint32_t reserved[2];
};
static_assert(sizeof(BlobHeader) == 64, "blob header is 64 bytes");

// A tensor inside the blob: `data` points at its first element; `elem` is the
// element size in bytes (2 = bf16 bits, 4 = float32).
struct TensorView {
  const void *data = nullptr;
  int64_t rows = 0, cols = 0;
  int elem = 4;
};

struct LayerViews {
  TensorView w_qkv, b_qkv, w_o, b_o, ln1_g, ln1_b, w_1, b_1, w_2, b_2, ln2_g, ln2_b;
};

struct ParsedBlob {
  BlobHeader h;
  TensorView tok_emb, pos_emb, norm_g, norm_b, head_w, head_b;
  std::vector<LayerViews> layers;
};

// Largest shapes the kernels are built for.
constexpr int kMaxHidden = 8192;
constexpr int kMaxHeadDim = 128;
constexpr int kMaxPos = 1024;

// Validate the header and sizes of `nbytes` bytes at `p` and fill `out`.
// Returns ES_OK or ES_ERR_FORMAT with a message.
es_status parse_blob(const void *p, int64_t nbytes, ParsedBlob *out);

}  // namespace es
