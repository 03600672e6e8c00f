// Launch wrappers for the gfx950 kernels of libencscore (host-callable).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "geometry.h"

namespace es {

// Device metadata of one packed batch (built on the host per call).
struct Ragged {
  const int32_t *off;    // [n_seqs + 1] token offsets, off[0] = 0
  const int64_t *sbase;  // [n_seqs] first element of sequence i's score blocks
  const int32_t *items;  // [2 * n_items] (sequence, first query row), kQTile rows each
  // [2 * n_sm_items] (sequence, first row) softmax work; the first
  // n_sm_narrow items have rows of at most 512 scores
  const int32_t *sm_items = nullptr;
  int32_t n_sm_narrow = 0;
  const int32_t *src = nullptr;   // [n_seqs] first id of sequence i in the id buffer (NULL: off)
  const int32_t *dest = nullptr;  // [n_seqs] reward slot of sequence i (NULL: i; < 0: none)
  // Shared prompts (causal models, fused attention only): sequence i continues
  // the plen[i] tokens at packed rows pref[i].. -- its positions start at
  // plen[i] and its queries also see those rows' keys and values.  NULL: none.
  const int32_t *pref = nullptr, *plen = nullptr;
  // Fused attention work, when split by length (NULL fused_items: every
  // entry of items runs on the one-wavefront kernel): fused_items [2 *
  // n_fused_items] (sequence, first query) 32-query tiles of short sequences,
  // mw_items [2 * n_mw_items] (sequence, first query) 128-query blocks of
  // sequences longer than kMwMinLen.
  const int32_t *fused_items = nullptr, *mw_items = nullptr;
  int32_t n_fused_items = 0, n_mw_items = 0;
  // Shared-prompt candidates (with plen): pfx_items [8 * n_pfx_items], four
  // (sequence, first query) 32-query tiles of candidates of one prompt per
  // entry (sequence < 0: empty slot; slot 0 never empty); those tiles are not
  // in fused_items / mw_items.
  const int32_t *pfx_items = nullptr;
  int32_t n_pfx_items = 0;
  int32_t n_seqs = 0, n_items = 0, max_len = 0, n_tokens = 0, n_sm_items = 0;
};

// ---- row kernels (rowops.hip)
// Embedding gather + position add (+ LayerNorm when `ln`): x fp32 [T, H];
// xb (bf16 bits or fp32, chosen by `act_bf16`) [T, ldb] when ln.
hipError_t launch_embed(bool w_bf16, bool act_bf16, bool ln, const int32_t *ids, const Ragged &r,
                        const void *tok, const void *pos, int vocab, int H, const float *g,
                        const float *b, float eps, float *x, void *xb, int ldb, int *flag,
                        hipStream_t st);
// Row LayerNorm of x (of x + sub when sub is non-NULL, both [rows, cols]):
// y fp32 [rows, cols] (nullable, may alias x or sub), yb [rows, ldb] (nullable;
// its columns [cols, pad_cols) are written with zeros, pad_cols <= ldb).
hipError_t launch_layernorm(bool act_bf16, const float *x, const float *sub, const float *g,
                            const float *b, int64_t rows, int cols, float eps, float *y, void *yb,
                            int ldb, int pad_cols, hipStream_t st);
// fp32 rows a [M, lda] (K columns, K a multiple of 16) into the
// split-operand layout; rows [M, 32 ceil(M / 32)) written as zeros.
hipError_t launch_split_rows(const float *a, int lda, int M, int K, uint16_t *out, hipStream_t st);
// LayerNorm of fp32 rows [rows, cols] (cols a multiple of 16) into the
// split-operand layout (device.h split_off): the input of a split GEMM.
hipError_t launch_layernorm_split(const float *x, const float *g, const float *b, int rows, int cols,
                                  float eps, uint16_t *out, hipStream_t st);
// Zero bytes [c0_bytes, c1_bytes) of each of `rows` rows of ld_bytes (all
// multiples of 4): the padding band of a K-padded GEMM operand.
hipError_t launch_zero_cols(void *base, int64_t ld_bytes, int rows, int64_t c0_bytes,
                            int64_t c1_bytes, hipStream_t st);
// Ragged softmax over score blocks: S fp32 -> P (bf16 bits or fp32).
hipError_t launch_softmax(bool p_bf16, const float *S, void *P, const Ragged &r, int n_heads,
                          bool causal, hipStream_t st);
// Row gather for the pruned last layer: a_dst row i = a_src row rows[i]
// (a_bytes per row, pitches in bytes), and the same for c; all sizes and
// pitches multiples of 4 bytes.
hipError_t launch_gather_rows(const void *a_src, int a_pitch, void *a_dst, int a_dpitch, int a_bytes,
                              const void *c_src, int c_pitch, void *c_dst, int c_dpitch, int c_bytes,
                              const int32_t *rows, int n, hipStream_t st);
// Best-of-N selection: best[p] = index (within prompt p's candidates
// cstart[p] .. cstart[p+1]-1) of the largest reward, the lowest among equals.
hipError_t launch_best_of_n(const float *rewards, const int32_t *cstart, int n_prompts,
                            int32_t *best, hipStream_t st);
// Reward head on the last token of each sequence (pre_ln: final LN first).
hipError_t launch_head(bool pre_ln, const float *x, int H, const Ragged &r, const float *g,
                       const float *b, float eps, const float *w, const float *hb, float offset,
                       float *rewards, hipStream_t st);

// ---- GEMMs (gemm.hip): out[m, n] = epi(sum_k A[m, k] W[n, k] + bias[n])
// kEpiResidualFfn behaves exactly like kEpiResidual; it is a separate kernel
// instance only so that profilers can tell the FFN2 GEMM from the
// attention-output GEMM.
enum Epilogue { kEpiBias = 0, kEpiGelu = 1, kEpiResidual = 2, kEpiF32 = 3, kEpiResidualFfn = 4 };
hipError_t launch_gemm_bf16(const uint16_t *A, int lda, const uint16_t *W, const float *bias,
                            const float *res, void *out, int ldc, int M, int N, int K, int epi,
                            hipStream_t st);
// The same with one tile configuration forced: 0 = 128 x 64 register-staged,
// 1 = 128 x 128 ping-pong, 2 = 256 x 256 ping-pong, 3 = 128 x 384 ping-pong,
// 4 = 32 x 64 register-staged, 5 = 256 x 256 software-pipelined, 6 = 32 x 32
// per wavefront fed straight from memory (latency tile).
constexpr int kGemmTiles = 7;
hipError_t launch_gemm_bf16_tile(int tile, const uint16_t *A, int lda, const uint16_t *W,
                                 const float *bias, const float *res, void *out, int ldc, int M,
                                 int N, int K, int epi, hipStream_t st);
// out = epi(A W^T + bias) with A [M, K] in the split-operand layout (each
// element a hi + lo bf16 pair, 16 significant bits; device.h split_off) and
// the bf16 weights, fp32 accumulation; K a multiple of 64.  epi kEpiF32 or
// kEpiResidual (res fp32 [M, ldc], may be out): fp32 rows in out; kEpiGelu:
// GELU(acc + bias) into outp in the split-operand layout with K' = N (N a
// multiple of 16), the next split GEMM's input.  A's row tiles are read
// whole (rows up to 32 ceil(M / 32)); outputs past M are not written.  For
// the last-token refinement of the reward rows.
hipError_t launch_gemm_split(const uint16_t *A, const uint16_t *W, const float *bias,
                             const float *res, float *out, uint16_t *outp, int ldc, int M, int N,
                             int K, int epi, hipStream_t st);
hipError_t launch_gemm_f32(const float *A, int lda, const float *W, const float *bias,
                           const float *res, float *out, int ldc, int M, int N, int K, int epi,
                           hipStream_t st);

// ---- attention (attn.hip).  qkv [T, ldq]: Q heads at columns h*dp, K at
// n_heads*dp + h*dp, V at 2*n_heads*dp + h*dp (dp = padded head dim).
hipError_t launch_scores(bool act_bf16, const void *qkv, int ldq, int n_heads, int dp, float scale,
                         bool causal, const Ragged &r, float *S, hipStream_t st);
hipError_t launch_pv(bool act_bf16, const void *P, const void *qkv, int ldq, int n_heads, int dp,
                     bool causal, const Ragged &r, void *ctx, int ldc, hipStream_t st);
// Fused attention (bf16): scores, online softmax and P.V in one kernel; the
// score rows never leave registers.
hipError_t launch_attn_fused(const uint16_t *qkv, int ldq, int n_heads, int dp, float scale,
                             bool causal, const Ragged &r, uint16_t *ctx, int ldc, hipStream_t st);
// Last-token refinement: for each sequence i of r, the attention of its last
// query in fp32 -- query and last key / value from row i of ql (fp32, pitch
// ldl, the bulk layout's Q | K | V columns), the other keys and values from
// the bulk bf16 qkv rows (shared-prompt rows first) -- into row i of ctx in
// the split-operand layout with K = kc (a multiple of 16); columns
// [n_heads dp, kc) zeroed.  Every sequence (prompt included) at most
// kLastMaxKeysHost positions (the weight blob's max_pos limit); a layout
// whose longest own sequence is longer is refused.
constexpr int kLastMaxKeysHost = 1024;
hipError_t launch_attn_last(const uint16_t *qkv, int ldq, const float *ql, int ldl, int n_heads,
                            int dp, float scale, const Ragged &r, uint16_t *ctx, int kc,
                            hipStream_t st);

}  // namespace es
