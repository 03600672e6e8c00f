// Launch wrappers for the gfx950 kernels of libencscore (host-callable).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace es {

// Query rows per attention work item; also the row tile of the softmax.
constexpr int kQTile = 32;

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

// Sequences longer than this (more than one query tile) run fused attention
// four query tiles per block.
constexpr int kMwMinLen = 32;
// Shared-prompt candidates of at most kPfxMaxLen tokens run four query tiles
// (of candidates of one prompt) per block when the prompt has at least
// kPfxMinPrompt tokens (two key tiles staged once for the block).
constexpr int kPfxMaxLen = 64;
constexpr int kPfxMinPrompt = 64;

// Softmax work geometry (shared by the host item builder and the kernel).
// A row of m scores is owned by G lanes, G the power of two covering its
// ceil(m / 8) eight-element chunks (at most 64; longer rows take several
// chunks per lane): each lane loads 8 scores as two float4 and stores its 8
// probabilities with one 16-byte bf16 store.  Bidirectional rows all have the
// sequence's length n, so one G serves all A * n rows of a sequence's block
// ([head][query] major) and items run across heads.  Causal row q has q + 1
// scores: rows are grouped by lane count -- q < 64 on 8 lanes, then 16, 32,
// and 64 lanes from q = 256 on -- so a lane group is at least half used,
// and an item never crosses a head or a lane-count boundary.  An item is up
// to kSoftmaxPasses (causal: kSoftmaxPassesCausal) passes of 4 wavefronts x
// (64 / G) rows.
constexpr int kSoftmaxPasses = 2;
constexpr int kSoftmaxPassesCausal = 8;
__host__ __device__ inline int softmax_lanes(int m) {
  const int nc = (m + 7) >> 3;
  int g = 1;
  while (g < nc && g < 64) g <<= 1;
  return g;
}
__host__ __device__ inline int softmax_row_lanes(int m, bool causal) {
  const int g = softmax_lanes(m);
  return causal && g < 8 ? 8 : g;
}
__host__ __device__ inline int softmax_rows_per_item(int g, bool causal) {
  return 4 * (64 / g) * (causal ? kSoftmaxPassesCausal : kSoftmaxPasses);
}
// The rows of one softmax item.  Bidirectional: rows r0 .. r0 + rows - 1
// of the sequence's A * n rows ([head][query] major).  Causal: rows qs ..
// qe - 1 of heads h0 .. h0 + hc - 1, all of one lane-count class; a class
// shorter than an item (the short rows near the diagonal's start) takes
// several heads per item, so every item moves a similar number of bytes.
// An item is named by its first row r0 = h0 n + qs.
struct SoftmaxItem {
  int g;         // lanes per row
  int rows;      // rows in the item
  int longest;   // scores of its longest row
  int h0, hc, qs, qe;
};
__host__ __device__ inline SoftmaxItem softmax_item(int r0, int n, int n_heads, bool causal) {
  SoftmaxItem it;
  if (!causal) {
    it.g = softmax_lanes(n);
    const int end = r0 + softmax_rows_per_item(it.g, false);
    it.rows = (end < n_heads * n ? end : n_heads * n) - r0;
    it.longest = n;
    it.h0 = it.hc = it.qs = it.qe = 0;
    return it;
  }
  const int h0 = r0 / n, q0 = r0 % n;
  const int g = softmax_row_lanes(q0 + 1, true);
  const int rpi = softmax_rows_per_item(g, true);
  const int cs = g <= 8 ? 0 : 4 * g;                  // class of rows needing g lanes
  int ce = g >= 64 ? n : 8 * g;
  if (ce > n) ce = n;
  it.g = g;
  it.h0 = h0;
  if (q0 == cs && ce - cs < rpi) {                    // whole class, several heads
    const int hc = rpi / (ce - cs);
    it.hc = hc < n_heads - h0 ? hc : n_heads - h0;
    it.qs = cs;
    it.qe = ce;
  } else {
    it.hc = 1;
    it.qs = q0;
    it.qe = q0 + rpi < ce ? q0 + rpi : ce;
  }
  it.rows = it.hc * (it.qe - it.qs);
  it.longest = it.qe;
  return it;
}
// First rows of the softmax items of one sequence, in order, with whether
// the item's longest row has more than 512 scores (needs more than one
// 8-score chunk per lane: such items run on a kernel with more registers,
// the rest on the lean one).
template <class F>
inline void softmax_items(int n, int n_heads, bool causal, F emit) {
  if (!causal) {
    for (int r0 = 0; r0 < n_heads * n;) {
      const SoftmaxItem it = softmax_item(r0, n, n_heads, false);
      emit(r0, it.longest > 512);
      r0 += it.rows;
    }
    return;
  }
  for (int cs = 0; cs < n;) {  // lane-count classes in order, heads inside
    const int g = softmax_row_lanes(cs + 1, true);
    const int ce = g >= 64 || 8 * g > n ? n : 8 * g;
    for (int h0 = 0; h0 < n_heads;) {
      int q = cs, hc = 1;
      while (q < ce) {
        const SoftmaxItem it = softmax_item(h0 * n + q, n, n_heads, true);
        emit(h0 * n + q, it.longest > 512);
        hc = it.hc;
        q = it.qe;
      }
      h0 += hc;
    }
    cs = ce;
  }
}

// Score-block row stride of a sequence of length n (elements).
__host__ __device__ inline int score_ld(int n) { return (n + 7) & ~7; }

// Score layout of the unfused attention: per sequence of length n and head
// h a block of score_block(n, causal) elements (heads back to back), row q
// of a block starting at score_row_off(q, n, causal).  Bidirectional: n rows
// of stride score_ld(n).  Causal: only the lower triangle, packed -- row q
// holds round_up(q + 1, 8) elements -- so the row reductions stream dense
// memory instead of half of every row:
//   sum_{r < q} round_up(r + 1, 8) = 8 (t + 1)(4 t + s),  q = 8 t + s.
__host__ __device__ inline int64_t score_row_off(int q, int n, bool causal) {
  if (!causal) return (int64_t)q * score_ld(n);
  const int64_t t = q >> 3, s = q & 7;
  return 8 * (t + 1) * (4 * t + s);
}
__host__ __device__ inline int64_t score_block(int n, bool causal) {
  return score_row_off(n, n, causal);
}

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
// 4 = 32 x 64 register-staged, 5 = 256 x 256 software-pipelined.
constexpr int kGemmTiles = 6;
hipError_t launch_gemm_bf16_tile(int tile, const uint16_t *A, int lda, const uint16_t *W,
                                 const float *bias, const float *res, void *out, int ldc, int M,
                                 int N, int K, int epi, hipStream_t st);
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

}  // namespace es
