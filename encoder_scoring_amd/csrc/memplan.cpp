// Host-only: offset planning for the sequence-length-aware workspace
// (TurboTransformers review, Proposed method: a memory allocator for
// variable-length inputs that balances footprint against allocation cost).
//
// Each intermediate tensor of a pass is a usage record (bytes, first and last
// step that touches it).  Two records may share addresses only if their step
// intervals are disjoint.  Records are placed largest first (ties: lower
// index first), each at the lowest aligned offset that overlaps no placed
// record whose interval meets its own; the arena needs max(offset + bytes).
// The sizes come from the pass's actual token count and score-block sizes,
// so the arena follows the lengths of the sequences being scored.
#include <algorithm>
#include <cinttypes>
#include <numeric>
#include <vector>

#include "common.h"
#include "memplan.h"

namespace es {

int64_t plan_arena(const std::vector<Usage> &u, int64_t align, std::vector<int64_t> &offset) {
  const size_t n = u.size();
  offset.assign(n, 0);
  std::vector<size_t> order(n);
  std::iota(order.begin(), order.end(), 0);
  std::stable_sort(order.begin(), order.end(),
                   [&](size_t a, size_t b) { return u[a].bytes > u[b].bytes; });
  std::vector<size_t> placed, hits;
  int64_t total = 0;
  for (size_t i : order) {
    const int64_t sz = round_up(u[i].bytes, align);
    if (sz == 0) continue;  // nothing to hold: offset 0, no conflict
    hits.clear();
    for (size_t j : placed)
      if (u[j].first <= u[i].last && u[i].first <= u[j].last) hits.push_back(j);
    std::sort(hits.begin(), hits.end(), [&](size_t a, size_t b) { return offset[a] < offset[b]; });
    int64_t at = 0;
    for (size_t j : hits) {
      if (at + sz <= offset[j]) break;  // the gap below record j holds it
      at = std::max(at, offset[j] + round_up(u[j].bytes, align));
    }
    offset[i] = at;
    placed.push_back(i);
    total = std::max(total, at + sz);
  }
  return total;
}

}  // namespace es

extern "C" es_status es_plan_arena(const int64_t *bytes, const int32_t *first_step,
                                   const int32_t *last_step, int32_t n, int64_t align,
                                   int64_t *offsets, int64_t *total) {
  using es::fail;
  if (n < 0 || !total || (n > 0 && (!bytes || !first_step || !last_step || !offsets)))
    return fail(ES_ERR_ARG, "es_plan_arena: bad arguments");
  if (align < 1 || (align & (align - 1)))
    return fail(ES_ERR_ARG, "es_plan_arena: align=%" PRId64 " is not a power of two", align);
  std::vector<es::Usage> u((size_t)n);
  for (int32_t i = 0; i < n; ++i) {
    if (bytes[i] < 0 || first_step[i] > last_step[i])
      return fail(ES_ERR_ARG, "es_plan_arena: record %d has bytes=%" PRId64 " steps [%d, %d]", i,
                  bytes[i], first_step[i], last_step[i]);
    u[i] = {bytes[i], first_step[i], last_step[i]};
  }
  std::vector<int64_t> off;
  *total = es::plan_arena(u, align, off);
  for (int32_t i = 0; i < n; ++i) offsets[i] = off[(size_t)i];
  es::clear_error();
  return ES_OK;
}
