// Host-side construction of the per-pass metadata of a scoring call, and a
// checker of every index it produces.  Plain C++ (no HIP): built into the GPU
// library and into the host-only library the CPU tests load.
//
// A pass packs one or more planned batches (TurboTransformers review,
// Proposed method: batches without fixed-length padding) back to back; its
// metadata is the token offsets, the score-block bases of the unfused
// attention, the attention and softmax work items, the id-source and
// reward-slot maps of a request stream, the shared-prompt rows of best-of-N
// ("Learning to summarize from human feedback", Method adaptation), and the
// last-token rows of the pruned last layer.
#include "layout.h"

#include <algorithm>
#include <cinttypes>
#include <cstdarg>
#include <cstring>

#include "geometry.h"

namespace es {

size_t push_bytes(std::vector<uint8_t> &buf, const void *p, size_t bytes) {
  const size_t at = (size_t)round_up((int64_t)buf.size(), 16);
  buf.resize(at + bytes);
  if (bytes) std::memcpy(buf.data() + at, p, bytes);
  return at;
}

es_status add_batch(const LayoutParams &p, std::vector<uint8_t> &meta,
                    std::vector<int32_t> &scratch, const int32_t *h_off, int32_t n,
                    const int32_t *src, const int32_t *dest, BatchLayout *L, int scale,
                    const int32_t *pref, const int32_t *plen) {
  L->scale = scale;
  if (!h_off) return fail(ES_ERR_ARG, "offsets pointer is NULL");
  if (n < 1) return fail(ES_ERR_ARG, "n_seqs=%d < 1", n);
  if (n > (int64_t)scale * p.max_seqs)
    return fail(ES_ERR_CAPACITY, "n_seqs=%d above max_seqs=%d", n, p.max_seqs);
  if (h_off[0] != 0) return fail(ES_ERR_ARG, "offsets[0]=%d, must be 0", h_off[0]);
  int max_len = 0;
  int64_t score = 0;
  std::vector<int64_t> sbase((size_t)n);
  for (int32_t i = 0; i < n; ++i) {
    const int64_t len = (int64_t)h_off[i + 1] - h_off[i];
    const int64_t np = plen ? plen[i] : 0;
    if (len < 1) return fail(ES_ERR_ARG, "offsets not strictly increasing at %d", i);
    if (np + len > p.P)
      return fail(ES_ERR_RANGE, "sequence %d has length %" PRId64 " > max_pos=%d", i, np + len, p.P);
    if (h_off[i + 1] > scale * p.max_tokens)
      return fail(ES_ERR_CAPACITY, "batch has more than max_tokens=%" PRId64 " tokens", p.max_tokens);
    max_len = std::max<int>(max_len, (int)len);
    // visible (query, key) pairs over the sequence's own queries
    L->pairs += (int64_t)p.A * (p.causal ? len * np + len * (len + 1) / 2 : len * len);
    sbase[i] = score;
    score += (int64_t)p.A * score_block((int)len, p.causal);
  }
  L->score_elems = score;
  if (!plen && score > scale * p.score_cap)
    return fail(ES_ERR_CAPACITY, "batch needs %" PRId64 " score elements (capacity %" PRId64 ")",
                score, p.score_cap);
  // attention work items, longest sequences first
  auto &ord = scratch;
  ord.resize(n);
  for (int32_t i = 0; i < n; ++i) ord[i] = i;
  auto keys_of = [&](int32_t i) { return h_off[i + 1] - h_off[i] + (plen ? plen[i] : 0); };
  std::stable_sort(ord.begin(), ord.end(), [&](int32_t a, int32_t b) { return keys_of(a) > keys_of(b); });
  std::vector<int32_t> items, sm_items, sm_wide, fitems, mitems, pitems;
  // shared-prompt candidates of up to kPfxMaxLen tokens whose prompt spans at
  // least kPfxMinPrompt positions: their 32-query tiles go four to a block,
  // grouped by prompt (all candidates of a prompt sort together: equal
  // prompt keys, then longest first), so the prompt's key tiles are staged
  // once per block
  auto pfx_tile = [&](int32_t i) {
    return plen && plen[i] >= kPfxMinPrompt && h_off[i + 1] - h_off[i] <= kPfxMaxLen;
  };
  if (plen)
    std::stable_sort(ord.begin(), ord.end(), [&](int32_t a, int32_t b) {
      const bool pa = pfx_tile(a), pb = pfx_tile(b);
      if (pa != pb) return pa < pb;
      if (pa && (plen[a] != plen[b] || pref[a] != pref[b]))
        return plen[a] != plen[b] ? plen[a] > plen[b] : pref[a] < pref[b];
      return keys_of(a) > keys_of(b);
    });
  int32_t pfx_slot = 0, pfx_np = -1, pfx_row = -1;
  for (int32_t sq : ord) {
    const int len = h_off[sq + 1] - h_off[sq];
    for (int q0 = 0; q0 < len; q0 += kQTile) {
      items.push_back(sq);
      items.push_back(q0);
    }
    if (pfx_tile(sq)) {
      if (plen[sq] != pfx_np || pref[sq] != pfx_row) {  // a new prompt starts a new block
        for (; pfx_slot % 4; ++pfx_slot) {
          pitems.push_back(-1);
          pitems.push_back(0);
        }
        pfx_np = plen[sq];
        pfx_row = pref[sq];
      }
      for (int q0 = 0; q0 < len; q0 += kQTile, ++pfx_slot) {
        pitems.push_back(sq);
        pitems.push_back(q0);
      }
    } else {
      // fused attention: long sequences in 128-query blocks (K, V staged once)
      auto &fl = len > kMwMinLen ? mitems : fitems;
      for (int q0 = 0; q0 < len; q0 += len > kMwMinLen ? 4 * kQTile : kQTile) {
        fl.push_back(sq);
        fl.push_back(q0);
      }
    }
    softmax_items(len, p.A, p.causal, [&](int r0, bool wide) {
      auto &dst = wide ? sm_wide : sm_items;
      dst.push_back(sq);
      dst.push_back(r0);
    });
  }
  auto &buf = meta;
  L->off = push_bytes(buf, h_off, sizeof(int32_t) * (n + 1));
  L->sbase = push_bytes(buf, sbase.data(), sizeof(int64_t) * n);
  L->items = push_bytes(buf, items.data(), sizeof(int32_t) * items.size());
  L->fitems = push_bytes(buf, fitems.data(), sizeof(int32_t) * fitems.size());
  L->mitems = push_bytes(buf, mitems.data(), sizeof(int32_t) * mitems.size());
  for (; pfx_slot % 4; ++pfx_slot) {
    pitems.push_back(-1);
    pitems.push_back(0);
  }
  L->pitems = push_bytes(buf, pitems.data(), sizeof(int32_t) * pitems.size());
  L->n_fitems = (int)(fitems.size() / 2);
  L->n_mitems = (int)(mitems.size() / 2);
  L->n_pitems = (int)(pitems.size() / 8);
  L->n_sm_narrow = (int)(sm_items.size() / 2);
  sm_items.insert(sm_items.end(), sm_wide.begin(), sm_wide.end());
  L->sm_items = push_bytes(buf, sm_items.data(), sizeof(int32_t) * sm_items.size());
  L->n_sm_items = (int)(sm_items.size() / 2);
  L->has_src = src != nullptr;
  L->has_dest = dest != nullptr;
  if (src) L->src = push_bytes(buf, src, sizeof(int32_t) * n);
  if (dest) L->dest = push_bytes(buf, dest, sizeof(int32_t) * n);
  {
    std::vector<int32_t> li((size_t)2 * n), lr((size_t)n), io((size_t)n + 1);
    for (int32_t i = 0; i < n; ++i) {
      const int32_t len = h_off[i + 1] - h_off[i];
      li[2 * i] = i;
      li[2 * i + 1] = len - 1;
      lr[i] = h_off[i + 1] - 1;
      io[i] = i;
      L->last_pairs += (int64_t)p.A * (p.causal ? len + (plen ? plen[i] : 0) : len);
    }
    io[n] = n;
    L->last_items = push_bytes(buf, li.data(), sizeof(int32_t) * li.size());
    L->last_rows = push_bytes(buf, lr.data(), sizeof(int32_t) * lr.size());
    L->iota = push_bytes(buf, io.data(), sizeof(int32_t) * io.size());
  }
  L->has_prefix = plen != nullptr;
  if (plen) {
    L->pref = push_bytes(buf, pref, sizeof(int32_t) * n);
    L->plen = push_bytes(buf, plen, sizeof(int32_t) * n);
  }
  L->n = n;
  L->n_items = (int)(items.size() / 2);
  L->max_len = max_len;
  L->n_tokens = h_off[n];
  return ES_OK;
}

es_status build_stream(const LayoutParams &p, const int32_t *lengths, int32_t n,
                       int64_t batch_overhead, int group, const std::vector<int64_t> &cost_table,
                       int32_t cost_max_batch, int32_t cost_max_len, std::vector<uint8_t> &meta,
                       std::vector<int32_t> &scratch, CallPlan *out) {
  if (!lengths || !out) return fail(ES_ERR_ARG, "NULL argument");
  if (n < 1) return fail(ES_ERR_ARG, "n=%d < 1", n);
  if (group < 1) return fail(ES_ERR_ARG, "group=%d < 1", group);
  es_status s;
  for (int32_t i = 0; i < n; ++i)
    if (lengths[i] < 1 || lengths[i] > p.P)
      return fail(ES_ERR_RANGE, "lengths[%d]=%d outside [1, max_pos=%d]", i, lengths[i], p.P);
  // a1: plan over the whole stream (host DP), budget = the workspace size
  std::vector<int32_t> order((size_t)n), starts((size_t)n + 1);
  int32_t nb = 0;
  int64_t cost = 0;
  if (cost_table.empty())
    s = es_plan_batches(lengths, n, p.max_tokens, batch_overhead, order.data(), starts.data(),
                        &nb, &cost);
  else  // the table's first max_seqs rows: no planned batch outgrows a workspace
    s = es_plan_batches_measured(lengths, n, p.max_tokens, cost_table.data(),
                                 std::min(cost_max_batch, p.max_seqs), cost_max_len,
                                 order.data(), starts.data(), &nb, &cost);
  if (s != ES_OK) return s;
  // request-order start of every sequence's ids in d_token_ids
  std::vector<int32_t> first((size_t)n);
  int64_t acc = 0;
  for (int32_t i = 0; i < n; ++i) {
    first[i] = (int32_t)acc;
    acc += lengths[i];
    if (acc > INT32_MAX) return fail(ES_ERR_RANGE, "more than INT32_MAX tokens in one call");
  }
  // a2: pack -- per batch, offsets over the plan order plus id-source and
  // reward-slot maps.  G consecutive planned batches (similar lengths, the
  // plan is sorted) are packed back to back into one layout and scored by one
  // pass through the layers: every kernel works per token or per sequence, so
  // a sequence's reward does not depend on which batches share the pass.
  const int G = group;
  const int32_t ng = (nb + G - 1) / G;
  meta.clear();
  out->passes.assign((size_t)ng, BatchLayout{});
  std::vector<int32_t> off, goff, src, dest;
  int64_t padded = 0;
  for (int32_t g = 0; g < ng; ++g) {
    // ng passes of as equal a batch count as possible (each at most G)
    const int32_t b0 = (int32_t)((int64_t)g * nb / ng), b1 = (int32_t)((int64_t)(g + 1) * nb / ng);
    goff.assign(1, 0);
    src.clear();
    dest.clear();
    for (int32_t b = b0; b < b1; ++b) {
      const int32_t lo = starts[b], hi = starts[b + 1], k = hi - lo;
      off.assign((size_t)k + 1, 0);
      if ((s = es_pack_offsets(lengths, order.data(), lo, hi, off.data())) != ES_OK) return s;
      const int32_t base = goff.back();
      for (int32_t j = 0; j < k; ++j) {
        goff.push_back(base + off[j + 1]);
        src.push_back(first[order[lo + j]]);
        dest.push_back(order[lo + j]);
      }
      padded += (int64_t)k * lengths[order[hi - 1]];
    }
    if ((s = add_batch(p, meta, scratch, goff.data(), (int32_t)dest.size(), src.data(), dest.data(), &out->passes[g],
                       b1 - b0)) != ES_OK)
      return s;
  }
  out->n_batches = nb;
  out->total_cost = cost;
  out->padded_tokens = padded;
  out->packed_tokens = acc;
  out->n_ids = acc;
  out->n_slots = n;
  return ES_OK;
}

es_status build_best_of_n(const LayoutParams &lp, const int32_t *prompt_lengths, int32_t n_prompts,
                          const int32_t *cand_lengths, const int32_t *cand_counts,
                          int64_t batch_overhead, int batches_per_pass, std::vector<uint8_t> &meta,
                          std::vector<int32_t> &scratch, CallPlan *out) {
  if (!prompt_lengths || !cand_lengths || !cand_counts || !out) return fail(ES_ERR_ARG, "NULL argument");
  if (n_prompts < 1) return fail(ES_ERR_ARG, "n_prompts=%d < 1", n_prompts);
  if (batches_per_pass < 1) return fail(ES_ERR_ARG, "batches_per_pass=%d < 1", batches_per_pass);
  es_status s;
  // per prompt: first candidate, token totals, group size (prompt + its candidates)
  std::vector<int32_t> cstart((size_t)n_prompts + 1, 0), group((size_t)n_prompts);
  std::vector<int64_t> pfirst((size_t)n_prompts), cfirst;
  int64_t ptok = 0;
  for (int32_t p = 0; p < n_prompts; ++p) {
    if (cand_counts[p] < 1) return fail(ES_ERR_ARG, "prompt %d has %d candidates", p, cand_counts[p]);
    if (prompt_lengths[p] < 1) return fail(ES_ERR_RANGE, "prompt %d has length %d", p, prompt_lengths[p]);
    cstart[p + 1] = cstart[p] + cand_counts[p];
    pfirst[p] = ptok;
    ptok += prompt_lengths[p];
  }
  const int32_t n_cand = cstart[n_prompts];
  cfirst.resize((size_t)n_cand);
  int64_t ctok = 0;
  for (int32_t p = 0; p < n_prompts; ++p) {
    int64_t g = prompt_lengths[p];
    for (int32_t c = cstart[p]; c < cstart[p + 1]; ++c) {
      const int32_t len = cand_lengths[c];
      if (len < 1 || (int64_t)prompt_lengths[p] + len > lp.P)
        return fail(ES_ERR_RANGE, "candidate %d: prompt %d + %d tokens outside [2, max_pos=%d]", c,
                    prompt_lengths[p], len, lp.P);
      cfirst[c] = ptok + ctok;
      ctok += len;
      g += len;
    }
    if (g > lp.max_tokens)
      return fail(ES_ERR_CAPACITY, "prompt %d with its candidates has %" PRId64 " tokens > max_tokens=%" PRId64,
                  p, g, lp.max_tokens);
    if (1 + cand_counts[p] > lp.max_seqs)
      return fail(ES_ERR_CAPACITY, "prompt %d has %d candidates (max_seqs=%d)", p, cand_counts[p], lp.max_seqs);
    group[p] = (int32_t)g;
  }
  if (ptok + ctok > INT32_MAX) return fail(ES_ERR_RANGE, "more than INT32_MAX tokens in one call");
  // a1: the planner over prompt groups, each an item as long as its tokens
  std::vector<int32_t> order((size_t)n_prompts), starts((size_t)n_prompts + 1);
  int32_t nb = 0;
  int64_t cost = 0;
  if ((s = es_plan_batches(group.data(), n_prompts, lp.max_tokens, batch_overhead, order.data(),
                           starts.data(), &nb, &cost)) != ES_OK)
    return s;
  // a2: per pass (G planned batches), every group as its prompt followed by
  // its candidates; a candidate continues its prompt's rows
  const int G = batches_per_pass;
  const int32_t ng = (nb + G - 1) / G;
  meta.clear();
  out->passes.assign((size_t)ng, BatchLayout{});
  std::vector<int32_t> off, src, dest, pref, plen;
  int64_t padded = 0;
  for (int32_t gi = 0; gi < ng; ++gi) {
    const int32_t b0 = (int32_t)((int64_t)gi * nb / ng), b1 = (int32_t)((int64_t)(gi + 1) * nb / ng);
    off.assign(1, 0);
    src.clear();
    dest.clear();
    pref.clear();
    plen.clear();
    for (int32_t b = b0; b < b1; ++b) {
      int32_t gmax = 0;
      for (int32_t k = starts[b]; k < starts[b + 1]; ++k) {
        const int32_t p = order[k];
        gmax = std::max(gmax, group[p]);
        const int32_t prow = off.back();
        off.push_back(prow + prompt_lengths[p]);
        src.push_back((int32_t)pfirst[p]);
        dest.push_back(-1);
        pref.push_back(0);
        plen.push_back(0);
        for (int32_t c = cstart[p]; c < cstart[p + 1]; ++c) {
          off.push_back(off.back() + cand_lengths[c]);
          src.push_back((int32_t)cfirst[c]);
          dest.push_back(c);
          pref.push_back(prow);
          plen.push_back(prompt_lengths[p]);
        }
      }
      padded += (int64_t)(starts[b + 1] - starts[b]) * gmax;
    }
    if ((s = add_batch(lp, meta, scratch, off.data(), (int32_t)dest.size(), src.data(), dest.data(), &out->passes[gi],
                       b1 - b0, pref.data(), plen.data())) != ES_OK)
      return s;
  }
  out->cand_starts = push_bytes(meta, cstart.data(), sizeof(int32_t) * cstart.size());
  out->n_batches = nb;
  out->total_cost = cost;
  out->padded_tokens = padded;
  out->packed_tokens = ptok + ctok;
  out->n_ids = ptok + ctok;
  out->n_slots = n_cand;
  return ES_OK;
}

// ---- checker

namespace {

struct Checker {
  int64_t bad = 0, checked = 0;
  std::string *first;
  void expect(bool ok, const char *fmt, ...) __attribute__((format(printf, 3, 4))) {
    ++checked;
    if (ok) return;
    if (bad++ == 0 && first) {
      char buf[512];
      va_list ap;
      va_start(ap, fmt);
      vsnprintf(buf, sizeof buf, fmt, ap);
      va_end(ap);
      *first = buf;
    }
  }
};

template <class T>
const T *at(const std::vector<uint8_t> &meta, size_t off, size_t count, Checker &c) {
  c.expect(off % alignof(T) == 0 && off + count * sizeof(T) <= meta.size(),
           "array at byte %zu (%zu elements) outside the %zu metadata bytes", off, count, meta.size());
  return reinterpret_cast<const T *>(meta.data() + off);
}

}  // namespace

int64_t check_pass(const LayoutParams &p, const std::vector<uint8_t> &meta, const BatchLayout &L,
                   int64_t n_ids, int32_t n_slots, int64_t *checked, std::string *first) {
  Checker c{0, 0, first};
  const int n = L.n, A = p.A;
  c.expect(n >= 1 && n <= (int64_t)L.scale * p.max_seqs, "pass of %d sequences", n);
  if (c.bad) return c.bad;
  const int32_t *off = at<int32_t>(meta, L.off, (size_t)n + 1, c);
  const int64_t *sbase = at<int64_t>(meta, L.sbase, (size_t)n, c);
  const int32_t *pref = L.has_prefix ? at<int32_t>(meta, L.pref, (size_t)n, c) : nullptr;
  const int32_t *plen = L.has_prefix ? at<int32_t>(meta, L.plen, (size_t)n, c) : nullptr;
  const int32_t *src = L.has_src ? at<int32_t>(meta, L.src, (size_t)n, c) : nullptr;
  const int32_t *dest = L.has_dest ? at<int32_t>(meta, L.dest, (size_t)n, c) : nullptr;
  if (c.bad) return c.bad;
  // token rows: packed, inside the pass's workspace rows
  c.expect(off[0] == 0 && off[n] == L.n_tokens, "offsets span [%d, %d), pass has %d tokens", off[0],
           off[n], L.n_tokens);
  c.expect(L.n_tokens <= (int64_t)L.scale * p.max_tokens, "pass of %d tokens over %d x %" PRId64,
           L.n_tokens, L.scale, p.max_tokens);
  int64_t score = 0;
  std::vector<int> len((size_t)n);
  for (int i = 0; i < n; ++i) {
    len[i] = off[i + 1] - off[i];
    const int np = plen ? plen[i] : 0;
    c.expect(len[i] >= 1 && np >= 0 && np + len[i] <= p.P, "sequence %d: %d tokens after a prompt of %d",
             i, len[i], np);
    c.expect(sbase[i] == score, "sequence %d: score base %" PRId64 ", expected %" PRId64, i, sbase[i], score);
    score += (int64_t)A * score_block(len[i], p.causal);
    if (src) c.expect(src[i] >= 0 && (int64_t)src[i] + len[i] <= n_ids,
                      "sequence %d reads ids [%d, %d) of %" PRId64, i, src[i], src[i] + len[i], n_ids);
    if (pref && np > 0) {  // the prompt is an earlier sequence of the pass with no reward slot
      int j = -1;
      for (int k = 0; k < i; ++k)
        if (off[k] == pref[i]) j = k;
      c.expect(j >= 0 && len[j] == np && (!dest || dest[j] < 0),
               "sequence %d: prompt rows [%d, %d) are not a prompt of the pass", i, pref[i], pref[i] + np);
    }
  }
  c.expect(score == L.score_elems, "score elements %" PRId64 ", layout says %" PRId64, score, L.score_elems);
  if (!L.has_prefix) c.expect(score <= (int64_t)L.scale * p.score_cap, "score elements over capacity");
  if (dest) {
    std::vector<char> seen((size_t)std::max(n_slots, 0), 0);
    for (int i = 0; i < n; ++i) {
      if (dest[i] < 0) continue;
      const bool ok = dest[i] < n_slots && !seen[dest[i]];
      c.expect(ok, "sequence %d writes reward slot %d of %d (or twice)", i, dest[i], n_slots);
      if (ok) seen[dest[i]] = 1;
    }
  }
  // attention work: every 32-query tile of every sequence exactly once
  std::vector<std::vector<char>> tiles((size_t)n);
  for (int i = 0; i < n; ++i) tiles[i].assign((size_t)(len[i] + kQTile - 1) / kQTile, 0);
  auto tile = [&](const char *what, int seq, int q0) {
    const bool ok = seq >= 0 && seq < n && q0 >= 0 && q0 < len[seq] && q0 % kQTile == 0;
    c.expect(ok, "%s item (%d, %d) outside the pass", what, seq, q0);
    return ok;
  };
  {
    const int32_t *it = at<int32_t>(meta, L.items, (size_t)2 * L.n_items, c);
    std::vector<std::vector<char>> seen = tiles;
    for (int k = 0; k < L.n_items && !c.bad; ++k)
      if (tile("attention", it[2 * k], it[2 * k + 1])) {
        char &s = seen[it[2 * k]][it[2 * k + 1] / kQTile];
        c.expect(!s, "attention tile (%d, %d) twice", it[2 * k], it[2 * k + 1]);
        s = 1;
      }
    for (int i = 0; i < n; ++i)
      for (char s : seen[i]) c.expect(s, "sequence %d has a query tile without an attention item", i);
  }
  {  // fused form: short tiles, 128-query blocks and shared-prompt blocks together
    std::vector<std::vector<char>> seen = tiles;
    auto mark = [&](const char *what, int seq, int q0, int span) {
      if (!tile(what, seq, q0)) return;
      for (int q = q0; q < std::min(q0 + span, len[seq]); q += kQTile) {
        char &s = seen[seq][q / kQTile];
        c.expect(!s, "fused tile (%d, %d) twice", seq, q);
        s = 1;
      }
    };
    const int32_t *f = at<int32_t>(meta, L.fitems, (size_t)2 * L.n_fitems, c);
    for (int k = 0; k < L.n_fitems && !c.bad; ++k) {
      c.expect(f[2 * k] < 0 || f[2 * k] >= n || len[f[2 * k]] <= kMwMinLen,
               "short-sequence item of %d tokens", f[2 * k] >= 0 && f[2 * k] < n ? len[f[2 * k]] : -1);
      mark("fused", f[2 * k], f[2 * k + 1], kQTile);
    }
    const int32_t *mw = at<int32_t>(meta, L.mitems, (size_t)2 * L.n_mitems, c);
    for (int k = 0; k < L.n_mitems && !c.bad; ++k) {
      c.expect(mw[2 * k + 1] % (4 * kQTile) == 0 &&
                   (mw[2 * k] < 0 || mw[2 * k] >= n || len[mw[2 * k]] > kMwMinLen),
               "128-query block at query %d", mw[2 * k + 1]);
      mark("four-tile", mw[2 * k], mw[2 * k + 1], 4 * kQTile);
    }
    const int32_t *px = at<int32_t>(meta, L.pitems, (size_t)8 * L.n_pitems, c);
    for (int k = 0; k < L.n_pitems && !c.bad; ++k) {
      c.expect(px[8 * k] >= 0, "shared-prompt block %d starts with an empty slot", k);
      for (int s = 0; s < 4; ++s) {
        const int seq = px[8 * k + 2 * s];
        if (seq < 0) continue;
        const int s0 = px[8 * k];
        c.expect(plen && s0 >= 0 && s0 < n && seq < n && pref[seq] == pref[s0] && plen[seq] == plen[s0],
                 "shared-prompt block %d mixes prompts", k);
        mark("shared-prompt", seq, px[8 * k + 2 * s + 1], kQTile);
      }
    }
    for (int i = 0; i < n; ++i)
      for (char s : seen[i]) c.expect(s, "sequence %d has a query tile without a fused item", i);
  }
  {  // softmax items: every (sequence, head, row) once, every score address in the buffer
    const int32_t *sm = at<int32_t>(meta, L.sm_items, (size_t)2 * L.n_sm_items, c);
    std::vector<std::vector<char>> rows((size_t)n);
    for (int i = 0; i < n; ++i) rows[i].assign((size_t)A * len[i], 0);
    for (int k = 0; k < L.n_sm_items && !c.bad; ++k) {
      const int seq = sm[2 * k], r0 = sm[2 * k + 1];
      if (!(seq >= 0 && seq < n && r0 >= 0 && r0 < A * len[seq])) {
        c.expect(false, "softmax item (%d, %d) outside the pass", seq, r0);
        continue;
      }
      const int m = len[seq];
      const SoftmaxItem it = softmax_item(r0, m, A, p.causal);
      c.expect((k < L.n_sm_narrow) == softmax_one_chunk(it.longest, p.causal),
               "softmax item %d on the wrong kernel", k);
      for (int i = 0; i < it.rows; ++i) {
        int h, q;
        if (p.causal) {
          h = it.h0 + i / (it.qe - it.qs);
          q = it.qs + i % (it.qe - it.qs);
        } else {
          h = (r0 + i) / m;
          q = (r0 + i) % m;
        }
        const bool in = h >= 0 && h < A && q >= 0 && q < m;
        c.expect(in, "softmax item (%d, %d) reaches head %d row %d", seq, r0, h, q);
        if (!in) continue;
        const int valid = p.causal ? q + 1 : m;
        const int cap = p.causal ? score_ld(q + 1) : score_ld(m);
        const int64_t last = sbase[seq] + (int64_t)h * score_block(m, p.causal) +
                             score_row_off(q, m, p.causal) + cap;
        c.expect(valid <= it.longest && it.g == (p.causal ? softmax_row_lanes(q + 1, true) : softmax_lanes(m)) &&
                     last <= L.score_elems,
                 "softmax row (%d, %d, %d) ends at element %" PRId64 " of %" PRId64, seq, h, q, last,
                 L.score_elems);
        char &s = rows[seq][(size_t)h * m + q];
        c.expect(!s, "softmax row (%d, %d, %d) twice", seq, h, q);
        s = 1;
      }
    }
    for (int i = 0; i < n; ++i)
      for (char s : rows[i]) c.expect(s, "sequence %d has a score row without a softmax item", i);
  }
  {  // pruned last layer: each sequence's last query and last token row
    const int32_t *li = at<int32_t>(meta, L.last_items, (size_t)2 * n, c);
    const int32_t *lr = at<int32_t>(meta, L.last_rows, (size_t)n, c);
    const int32_t *io = at<int32_t>(meta, L.iota, (size_t)n + 1, c);
    for (int i = 0; i < n && !c.bad; ++i) {
      c.expect(li[2 * i] == i && li[2 * i + 1] == len[i] - 1, "last-query item %d is (%d, %d)", i,
               li[2 * i], li[2 * i + 1]);
      c.expect(lr[i] == off[i + 1] - 1 && lr[i] < L.n_tokens, "last row of sequence %d is %d", i, lr[i]);
      c.expect(io[i] == i, "compacted offsets of the last rows");
    }
  }
  if (checked) *checked += c.checked;
  return c.bad;
}

}  // namespace es

// Host-only: the checks above over every pass of a call's plan.
extern "C" es_status es_check_plan(const int32_t *lengths, int32_t n, const int32_t *prompt_lengths,
                                   const int32_t *cand_counts, int32_t n_prompts, int32_t n_heads,
                                   int32_t causal, int32_t max_pos, int64_t max_tokens,
                                   int32_t max_seqs, int64_t batch_overhead,
                                   int32_t batches_per_pass, int64_t *n_passes, int64_t *n_checked,
                                   int64_t *n_violations) {
  using namespace es;
  if (!lengths || !n_checked || !n_violations || !n_passes) return fail(ES_ERR_ARG, "NULL argument");
  if (n_heads < 1 || max_pos < 1 || max_tokens < 1 || max_seqs < 1 || (causal != 0 && causal != 1))
    return fail(ES_ERR_ARG, "bad model shape");
  LayoutParams p;
  p.A = n_heads;
  p.causal = causal != 0;
  p.P = max_pos;
  p.max_tokens = max_tokens;
  p.max_seqs = max_seqs;
  p.score_cap = (int64_t)n_heads * max_tokens * score_ld((int)std::min<int64_t>(max_pos, max_tokens));
  std::vector<uint8_t> meta;
  std::vector<int32_t> scratch;
  CallPlan plan;
  es_status s;
  if (n_prompts > 0) {
    if (!prompt_lengths || !cand_counts) return fail(ES_ERR_ARG, "NULL prompt arrays");
    s = build_best_of_n(p, prompt_lengths, n_prompts, lengths, cand_counts, batch_overhead,
                        batches_per_pass, meta, scratch, &plan);
  } else {
    s = build_stream(p, lengths, n, batch_overhead, batches_per_pass, std::vector<int64_t>(), 0, 0,
                     meta, scratch, &plan);
  }
  if (s != ES_OK) return s;
  int64_t bad = 0, checked = 0;
  std::string first;
  for (const BatchLayout &L : plan.passes) {
    std::string f;
    const int64_t b = check_pass(p, meta, L, plan.n_ids, plan.n_slots, &checked, &f);
    if (b && first.empty()) first = f;
    bad += b;
  }
  *n_passes = (int64_t)plan.passes.size();
  *n_checked = checked;
  *n_violations = bad;
  if (bad) return fail(ES_ERR_FORMAT, "%" PRId64 " violations; first: %s", bad, first.c_str());
  clear_error();
  return ES_OK;
}
