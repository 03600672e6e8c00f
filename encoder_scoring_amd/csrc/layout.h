// Host-side construction of the per-pass metadata of a scoring call
// (layout.cpp).  No HIP: the same code builds into the GPU library and the
// host-only library, so the CPU tests can check every index it produces.
#pragma once

#include <cstddef>
#include <cstdint>
#include <string>
#include <vector>

#include "common.h"

namespace es {

// What the metadata depends on: the model's shape and the handle's capacity.
struct LayoutParams {
  int A = 0;               // attention heads
  bool causal = false;
  int P = 0;               // max positions (longest sequence, prompt included)
  int64_t max_tokens = 0;  // tokens of one planned batch
  int max_seqs = 0;        // sequences of one planned batch
  int64_t score_cap = 0;   // score elements of one planned batch (fixed workspace)
};

// One pass's metadata: byte offsets of its arrays inside the call's
// metadata buffer (uploaded in one copy), and their sizes.
struct BatchLayout {
  size_t off = 0, sbase = 0, items = 0, sm_items = 0, src = 0, dest = 0, pref = 0, plen = 0;
  size_t fitems = 0, mitems = 0, pitems = 0;  // fused attention split by length (es::Ragged)
  int n_fitems = 0, n_mitems = 0, n_pitems = 0;
  size_t last_items = 0, last_rows = 0, iota = 0;  // last-token work of the pruned last layer
  int64_t last_pairs = 0;  // visible (query, key) pairs of the last queries, over heads
  bool has_src = false, has_dest = false, has_prefix = false;
  int n = 0, n_items = 0, n_sm_items = 0, n_sm_narrow = 0, max_len = 0, n_tokens = 0;
  int scale = 1;            // planned batches in the pass
  int64_t pairs = 0;        // visible (query, key) pairs summed over heads
  int64_t score_elems = 0;  // ragged score-block elements (unfused attention)
};

// Append `bytes` at the next 16-byte boundary of `buf`; returns the offset.
size_t push_bytes(std::vector<uint8_t> &buf, const void *p, size_t bytes);

// Validate one pass given by its host offsets (n sequences, `scale` planned
// batches) and append its metadata to `meta`.  src / dest (nullable): first
// id of each sequence in the id buffer / its reward slot (< 0: none).
// pref / plen (both or neither): sequence i continues the plen[i] tokens at
// packed rows pref[i].. (a shared prompt).
es_status add_batch(const LayoutParams &p, std::vector<uint8_t> &meta,
                    std::vector<int32_t> &scratch, const int32_t *h_off, int32_t n,
                    const int32_t *src, const int32_t *dest, BatchLayout *L, int scale = 1,
                    const int32_t *pref = nullptr, const int32_t *plen = nullptr);

// A planned call: its passes and plan statistics.
struct CallPlan {
  std::vector<BatchLayout> passes;
  int32_t n_batches = 0;
  int64_t total_cost = 0, padded_tokens = 0, packed_tokens = 0;
  int64_t n_ids = 0;       // length of the id buffer the call reads
  int32_t n_slots = 0;     // reward slots it writes
  size_t cand_starts = 0;  // best-of-N: offset of the per-prompt candidate starts
};

// es_score_requests' host work: plan the stream (linear cost, or the cost
// table when non-empty, its first cost_max_batch rows), pack groups of
// `group` planned batches into passes, lay out each pass.
es_status build_stream(const LayoutParams &p, const int32_t *lengths, int32_t n,
                       int64_t batch_overhead, int group, const std::vector<int64_t> &cost_table,
                       int32_t cost_max_batch, int32_t cost_max_len, std::vector<uint8_t> &meta,
                       std::vector<int32_t> &scratch, CallPlan *out);

// es_score_best_of_n's host work: plan prompt groups (a prompt and all its
// candidates) and lay out each pass as prompts followed by their candidates.
es_status build_best_of_n(const LayoutParams &lp, const int32_t *prompt_lengths, int32_t n_prompts,
                          const int32_t *cand_lengths, const int32_t *cand_counts,
                          int64_t batch_overhead, int batches_per_pass, std::vector<uint8_t> &meta,
                          std::vector<int32_t> &scratch, CallPlan *out);

// Check every index of one pass's metadata against the buffer it addresses
// (token rows, score elements, id buffer, reward slots, work-item coverage).
// Returns the number of violations; the first is described in *first.
int64_t check_pass(const LayoutParams &p, const std::vector<uint8_t> &meta, const BatchLayout &L,
                   int64_t n_ids, int32_t n_slots, int64_t *checked, std::string *first);

}  // namespace es
