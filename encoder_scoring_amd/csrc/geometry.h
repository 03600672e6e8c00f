// Work geometry shared by the host-side metadata builder (layout.cpp, also
// built with a plain C++ compiler) and the gfx950 kernels: query tiles,
// fused-attention splits, the softmax work items and the ragged score
// layout of the unfused attention.
#pragma once

#include <cstdint>

#if defined(__HIP__)
#define ES_HD __host__ __device__
#else
#define ES_HD
#endif

namespace es {

// Query rows per attention work item; also the row tile of the softmax.
constexpr int kQTile = 32;


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
// scores: rows are grouped by lane count -- q < 64 on 8 lanes, then 16, 32
// and 64 lanes up to 512 scores -- so a lane group is at least half used, and
// an item never crosses a head or a lane-count boundary.  Causal rows of 513
// to 1024 scores take G = 128 lanes, two wavefronts of one chunk each,
// which combine their max and sum through LDS: they stay on the lean
// one-chunk kernel (as a launch of their own, with three chunks on 32 lanes,
// those rows were a single round of latency-bound blocks).  Longer causal
// rows take 64 lanes and several chunks each.  An item is up to
// kSoftmaxPasses (causal: kSoftmaxPassesCausal) passes of the block's 4
// wavefronts, 256 / G rows per pass.
constexpr int kSoftmaxPasses = 2;
constexpr int kSoftmaxPassesCausal = 8;
ES_HD inline int softmax_lanes(int m) {
  const int nc = (m + 7) >> 3;
  int g = 1;
  while (g < nc && g < 64) g <<= 1;
  return g;
}
ES_HD inline int softmax_row_lanes(int m, bool causal) {
  if (causal && m > 512 && m <= 1024) return 128;
  const int g = softmax_lanes(m);
  return causal && g < 8 ? 8 : g;
}
// The causal lane-count class of row q of a sequence of n: rows [cs, ce)
// all take softmax_row_lanes(q + 1) lanes.
ES_HD inline void softmax_causal_class(int q, int n, int &cs, int &ce) {
  const int m = q + 1;
  if (m <= 64) cs = 0, ce = 64;
  else if (m <= 128) cs = 64, ce = 128;
  else if (m <= 256) cs = 128, ce = 256;
  else if (m <= 512) cs = 256, ce = 512;
  else if (m <= 1024) cs = 512, ce = 1024;
  else cs = 1024, ce = n;
  if (ce > n) ce = n;
}
ES_HD inline int softmax_rows_per_item(int g, bool causal) {
  return (256 / g) * (causal ? kSoftmaxPassesCausal : kSoftmaxPasses);
}
// Items whose rows take one eight-score chunk per lane (at most 512 scores,
// or a causal row of at most 1024 on two wavefronts) run on the lean kernel.
ES_HD inline bool softmax_one_chunk(int longest, bool causal) {
  return longest <= (causal ? 1024 : 512);
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
ES_HD inline SoftmaxItem softmax_item(int r0, int n, int n_heads, bool causal) {
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
  int cs, ce;                                         // class of rows needing g lanes
  softmax_causal_class(q0, n, cs, ce);
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
// the item's rows need more than one 8-score chunk per lane (such items run
// on a kernel with more registers, the rest on the lean one).
template <class F>
inline void softmax_items(int n, int n_heads, bool causal, F emit) {
  if (!causal) {
    for (int r0 = 0; r0 < n_heads * n;) {
      const SoftmaxItem it = softmax_item(r0, n, n_heads, false);
      emit(r0, !softmax_one_chunk(it.longest, false));
      r0 += it.rows;
    }
    return;
  }
  for (int cs = 0; cs < n;) {  // lane-count classes in order, heads inside
    int c0, ce;
    softmax_causal_class(cs, n, c0, ce);  // c0 == cs
    for (int h0 = 0; h0 < n_heads;) {
      int q = cs, hc = 1;
      while (q < ce) {
        const SoftmaxItem it = softmax_item(h0 * n + q, n, n_heads, true);
        emit(h0 * n + q, !softmax_one_chunk(it.longest, true));
        hc = it.hc;
        q = it.qe;
      }
      h0 += hc;
    }
    cs = ce;
  }
}

// Score-block row stride of a sequence of length n (elements).
ES_HD inline int score_ld(int n) { return (n + 7) & ~7; }

// Score layout of the unfused attention: per sequence of length n and head
// h a block of score_block(n, causal) elements (heads back to back), row q
// of a block starting at score_row_off(q, n, causal).  Bidirectional: n rows
// of stride score_ld(n).  Causal: only the lower triangle, packed -- row q
// holds round_up(q + 1, 8) elements -- so the row reductions stream dense
// memory instead of half of every row:
//   sum_{r < q} round_up(r + 1, 8) = 8 (t + 1)(4 t + s),  q = 8 t + s.
ES_HD inline int64_t score_row_off(int q, int n, bool causal) {
  if (!causal) return (int64_t)q * score_ld(n);
  const int64_t t = q >> 3, s = q & 7;
  return 8 * (t + 1) * (4 * t + s);
}
ES_HD inline int64_t score_block(int n, bool causal) {
  return score_row_off(n, n, causal);
}

}  // namespace es
