// Host-only part of libencscore: error strings, the batch planner and offset
// packing.  Nothing here touches HIP, so it also builds with g++ alone.
//
// Planner: TurboTransformers review (Abstract; Proposed method) -- requests
// are sorted by length and grouped by a dynamic-programming batch scheduler
// with minimal padding.  Cost reading: sum over batches of
// (overhead + |B| * max_len(B)) under |B| * max_len(B) <= max_tokens.  In
// sorted order a batch [j, i) pads to (i - j) * s[i-1], so
//   f[i] = min_{j: (i-j)*s[i-1] <= T} f[j] + c + (i - j) * s[i-1],
// and since s is ascending only j >= i - floor(T / s[i-1]) are feasible.
#include <algorithm>
#include <cinttypes>
#include <cstring>
#include <limits>
#include <numeric>
#include <vector>

#include "common.h"

namespace es {

static thread_local std::string g_last_error;

es_status fail(es_status code, const char *fmt, ...) {
  char buf[1024];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

void clear_error() { g_last_error.clear(); }

}  // namespace es

extern "C" const char *es_last_error(void) { return es::g_last_error.c_str(); }

extern "C" const char *es_version(void) { return "encscore 0.1 (gfx950)"; }

extern "C" es_status es_plan_batches(const int32_t *lengths, int32_t n, int64_t max_tokens,
                                     int64_t batch_overhead, int32_t *order,
                                     int32_t *batch_starts, int32_t *n_batches,
                                     int64_t *total_cost) {
  using es::fail;
  if (n < 0) return fail(ES_ERR_ARG, "es_plan_batches: n=%d < 0", n);
  if (!batch_starts || !n_batches || !total_cost || (n > 0 && (!lengths || !order)))
    return fail(ES_ERR_ARG, "es_plan_batches: NULL pointer");
  if (max_tokens < 1) return fail(ES_ERR_ARG, "es_plan_batches: max_tokens=%" PRId64 " < 1", max_tokens);
  if (batch_overhead < 0)
    return fail(ES_ERR_ARG, "es_plan_batches: batch_overhead=%" PRId64 " < 0", batch_overhead);
  for (int32_t i = 0; i < n; ++i) {
    if (lengths[i] < 1 || (int64_t)lengths[i] > max_tokens)
      return fail(ES_ERR_RANGE, "es_plan_batches: lengths[%d]=%d outside [1, %" PRId64 "]", i,
                  lengths[i], max_tokens);
  }
  // every f[i] <= i * (c + T); refuse inputs whose cost could overflow int64
  const int64_t lim = std::numeric_limits<int64_t>::max() / 4;
  if (n > 0 && (batch_overhead > lim / n || max_tokens > lim / n ||
                (batch_overhead + max_tokens) > lim / n))
    return fail(ES_ERR_RANGE, "es_plan_batches: overhead/max_tokens too large for int64 costs");

  std::vector<int32_t> idx(n);
  std::iota(idx.begin(), idx.end(), 0);
  std::stable_sort(idx.begin(), idx.end(),
                   [&](int32_t a, int32_t b) { return lengths[a] < lengths[b]; });
  std::vector<int64_t> f(n + 1, 0);
  std::vector<int32_t> arg(n + 1, 0);
  for (int32_t i = 1; i <= n; ++i) {
    const int64_t L = lengths[idx[i - 1]];
    const int64_t kmax = max_tokens / L;  // >= 1 since L <= max_tokens
    const int32_t jlo = (int32_t)std::max<int64_t>(0, (int64_t)i - kmax);
    int64_t best = std::numeric_limits<int64_t>::max();
    int32_t bj = jlo;
    for (int32_t j = jlo; j < i; ++j) {
      const int64_t v = f[j] + batch_overhead + (int64_t)(i - j) * L;
      if (v < best) {  // strict: the first (smallest) minimising j wins
        best = v;
        bj = j;
      }
    }
    f[i] = best;
    arg[i] = bj;
  }
  // backtrack the split points
  std::vector<int32_t> starts;
  for (int32_t i = n; i > 0; i = arg[i]) starts.push_back(i);
  starts.push_back(0);
  std::reverse(starts.begin(), starts.end());
  if (n > 0) std::memcpy(order, idx.data(), sizeof(int32_t) * n);
  std::memcpy(batch_starts, starts.data(), sizeof(int32_t) * starts.size());
  *n_batches = (int32_t)starts.size() - 1;
  *total_cost = f[n];
  es::clear_error();
  return ES_OK;
}

// Measured-cost planner: the cost of a batch is a table entry
// C[|B|-1][max_len(B)-1] (e.g. the measured latency of |B| sequences of that
// length) in place of overhead + |B| * max_len.  With every row of C
// non-decreasing in the length, contiguous batches of the sorted order stay
// optimal over all partitions, so the same prefix DP applies:
//   f[i] = min_{j: i-j <= max_batch, (i-j)*s[i-1] <= T} f[j] + C[i-j-1][s[i-1]-1].
extern "C" es_status es_plan_batches_measured(const int32_t *lengths, int32_t n,
                                              int64_t max_tokens, const int64_t *cost_table,
                                              int32_t max_batch, int32_t max_len,
                                              int32_t *order, int32_t *batch_starts,
                                              int32_t *n_batches, int64_t *total_cost) {
  using es::fail;
  if (n < 0) return fail(ES_ERR_ARG, "es_plan_batches_measured: n=%d < 0", n);
  if (!batch_starts || !n_batches || !total_cost || !cost_table || (n > 0 && (!lengths || !order)))
    return fail(ES_ERR_ARG, "es_plan_batches_measured: NULL pointer");
  if (max_tokens < 1)
    return fail(ES_ERR_ARG, "es_plan_batches_measured: max_tokens=%" PRId64 " < 1", max_tokens);
  if (max_batch < 1 || max_len < 1 || (int64_t)max_batch * max_len > (int64_t)1 << 28)
    return fail(ES_ERR_ARG, "es_plan_batches_measured: table %d x %d outside [1, 2^28] entries",
                max_batch, max_len);
  const int64_t lim = std::numeric_limits<int64_t>::max() / 4 / std::max<int32_t>(n, 1);
  for (int32_t b = 0; b < max_batch; ++b) {
    const int64_t *row = cost_table + (size_t)b * max_len;
    for (int32_t l = 0; l < max_len; ++l) {
      if (row[l] < 0 || row[l] > lim)
        return fail(ES_ERR_ARG, "es_plan_batches_measured: C[%d][%d]=%" PRId64 " outside [0, %" PRId64 "]",
                    b, l, row[l], lim);
      if (l > 0 && row[l] < row[l - 1])
        return fail(ES_ERR_ARG, "es_plan_batches_measured: row %d falls from %" PRId64 " to %" PRId64
                    " at length %d (rows must be non-decreasing in the length)", b, row[l - 1], row[l], l + 1);
    }
  }
  for (int32_t i = 0; i < n; ++i) {
    if (lengths[i] < 1 || (int64_t)lengths[i] > max_tokens || lengths[i] > max_len)
      return fail(ES_ERR_RANGE, "es_plan_batches_measured: lengths[%d]=%d outside [1, min(%" PRId64 ", %d)]",
                  i, lengths[i], max_tokens, max_len);
  }
  std::vector<int32_t> idx(n);
  std::iota(idx.begin(), idx.end(), 0);
  std::stable_sort(idx.begin(), idx.end(),
                   [&](int32_t a, int32_t b) { return lengths[a] < lengths[b]; });
  std::vector<int64_t> f(n + 1, 0);
  std::vector<int32_t> arg(n + 1, 0);
  for (int32_t i = 1; i <= n; ++i) {
    const int32_t L = lengths[idx[i - 1]];
    const int64_t kmax = std::min<int64_t>(max_tokens / L, max_batch);  // >= 1
    const int32_t jlo = (int32_t)std::max<int64_t>(0, (int64_t)i - kmax);
    const int64_t *col = cost_table + (L - 1);  // C[size-1][L-1] = col[(size-1) * max_len]
    int64_t best = std::numeric_limits<int64_t>::max();
    int32_t bj = jlo;
    for (int32_t j = jlo; j < i; ++j) {
      const int64_t v = f[j] + col[(size_t)(i - j - 1) * max_len];
      if (v < best) {  // strict: the first (smallest) minimising j wins
        best = v;
        bj = j;
      }
    }
    f[i] = best;
    arg[i] = bj;
  }
  std::vector<int32_t> starts;
  for (int32_t i = n; i > 0; i = arg[i]) starts.push_back(i);
  starts.push_back(0);
  std::reverse(starts.begin(), starts.end());
  if (n > 0) std::memcpy(order, idx.data(), sizeof(int32_t) * n);
  std::memcpy(batch_starts, starts.data(), sizeof(int32_t) * starts.size());
  *n_batches = (int32_t)starts.size() - 1;
  *total_cost = f[n];
  es::clear_error();
  return ES_OK;
}

extern "C" es_status es_pack_offsets(const int32_t *lengths, const int32_t *order, int32_t begin,
                                     int32_t end, int32_t *offsets) {
  using es::fail;
  if (!offsets || begin < 0 || end < begin || (end > begin && (!lengths || !order)))
    return fail(ES_ERR_ARG, "es_pack_offsets: bad arguments (begin=%d end=%d)", begin, end);
  int64_t acc = 0;
  offsets[0] = 0;
  for (int32_t k = begin; k < end; ++k) {
    const int32_t len = lengths[order[k]];
    if (len < 1) return fail(ES_ERR_RANGE, "es_pack_offsets: length %d < 1", len);
    acc += len;
    if (acc > std::numeric_limits<int32_t>::max())
      return fail(ES_ERR_RANGE, "es_pack_offsets: total above INT32_MAX");
    offsets[k - begin + 1] = (int32_t)acc;
  }
  return ES_OK;
}
