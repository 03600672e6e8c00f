// Model handle, weight upload, per-batch metadata and the forward pass.
//
// Data layout in HBM (T = packed tokens of one batch, no padding between
// sequences; every buffer is sized once for max_tokens rounded up to 256 rows):
//   x     fp32 [T, H]        residual stream (post-LN: LayerNorm outputs)
//   y     fp32 [T, H]        GEMM + residual output before a post-LN LayerNorm
//   xb    act  [T, Hp]       GEMM input copy of the normalised rows
//   qkv   act  [T, 3*A*dp]   Q | K | V, head h at columns h*dp of each part
//   ctx   act  [T, Kc]       attention context, head h at columns h*dp
//   hmid  act  [T, Fp]       GELU(FFN1)
//   S     fp32 ragged        per (sequence, head) score blocks: n x ld, or the packed
//                            lower triangle when causal (score_row_off)
//   P     act  ragged        softmax output, same indexing as S
// act = bf16 for bf16 models (fp32 accumulation everywhere), fp32 otherwise.
// Hp, Kc, Fp round widths up to 64 (zero columns); dp rounds the head dim up
// to a power of two >= 32 by inserting zero rows into W_qkv and zero columns
// into W_o, which leaves every result unchanged.
#include <algorithm>
#include <chrono>
#include <cinttypes>
#include <cmath>
#include <cstring>
#include <fstream>
#include <mutex>
#include <vector>

#include "blob.h"
#include "common.h"
#include "kernels.h"
#include "layout.h"
#include "memplan.h"

// Scratch of es_score_batch_static, the entry point that allocates nothing:
// every intermediate of its pass (uploaded batch metadata, activations, score
// blocks) lives here.  Each GPU the library's code is loaded on holds its own
// copy until the process ends; host code reaches a device's copy only through
// the address hipGetSymbolAddress returns for it (static_scratch_of below).
static __device__ __align__(256) char scratch[ES_STATIC_SCRATCH_BYTES];

namespace {

using es::fail;
using es::round_up;
using es::BatchLayout;
using es::push_bytes;

#define HIP_TRY(expr)                                                                     \
  do {                                                                                    \
    hipError_t _e = (expr);                                                               \
    if (_e != hipSuccess)                                                                 \
      return fail(ES_ERR_HIP, "%s failed: %s (%s:%d)", #expr, hipGetErrorString(_e),      \
                  __FILE__, __LINE__);                                                    \
  } while (0)

struct DevLayer {
  void *w_qkv = nullptr, *w_o = nullptr, *w_1 = nullptr, *w_2 = nullptr;
  float *b_qkv = nullptr, *b_o = nullptr, *ln1_g = nullptr, *ln1_b = nullptr;
  float *b_1 = nullptr, *b_2 = nullptr, *ln2_g = nullptr, *ln2_b = nullptr;
};

int pow2_at_least(int v) {
  int p = 32;
  while (p < v) p <<= 1;
  return p;
}

}  // namespace

struct es_model {
  // shape
  int L = 0, H = 0, A = 0, d = 0, dp = 0, F = 0, V = 0, P = 0;
  bool pre_ln = false, causal = false, bf16 = false;
  float eps = 0.f, offset = 0.f;
  int Hp = 0, Nqkv = 0, Kc = 0, Fp = 0;
  // capacity
  int64_t max_tokens = 0, Tcap = 0, score_cap = 0;
  int attn_mode = 0;  // 0: scores -> softmax -> P.V, 1: fused (the bf16 default, set in build)
  // last-token refinement of the reward rows: refine_ok where the model
  // supports it (pre-LN bf16, set in build), refine whether it runs
  // (es_set_refinement, default refine_ok)
  bool refine_ok = false, refine = false;
  int max_seqs = 0;
  int device = 0;
  // weights
  void *tok_emb = nullptr, *pos_emb = nullptr;
  float *norm_g = nullptr, *norm_b = nullptr, *head_w = nullptr, *head_b = nullptr;
  std::vector<DevLayer> layers;
  // workspaces: one per batch in flight (es_set_concurrency)
  struct Workspace {
    int scale = 0;  // fixed buffers: capacity in planned batches (tokens, sequences, score elements)
    float *x = nullptr, *y = nullptr, *S = nullptr;
    void *xb = nullptr, *qkv = nullptr, *ctx = nullptr, *hmid = nullptr, *Pb = nullptr;
    float *ref = nullptr;  // last-token refinement rows (refine_floats per sequence)
    hipStream_t stream = nullptr;  // internal stream used when several batches are in flight
    hipEvent_t done = nullptr;
    // length-aware memory: one arena; the tensors above point into it per pass
    char *arena = nullptr;
    int64_t arena_cap = 0;
    int64_t call_need = 0, prev_call_need = 0;  // largest pass need of this / the last call
    bool first_in_call = false;
  };
  int mem_mode = 1;  // ES_MEM_FIXED / ES_MEM_LENGTH_AWARE / ES_MEM_EXACT (es_set_memory_mode)
  int64_t work_allocs = 0, peak_work = 0;  // workspace / arena allocations, largest total held
  double work_alloc_ms = 0.0;                // host time spent allocating them
  std::vector<Workspace> ws;  // allocated workspaces; the first `lanes` are used
  int lanes = 1;
  int group = 1;  // planned batches scored by one pass through the layers
  // measured batch costs for es_score_requests' planner (es_set_cost_table);
  // empty: the linear cost overhead + |B| * max_len
  std::vector<int64_t> cost_table;
  int32_t cost_max_batch = 0, cost_max_len = 0;
  bool prune = true;  // last layer on the last token of each sequence only (es_set_pruning)
  hipEvent_t fork_ev = nullptr;
  // the last-token refinement's own stream (used with one pass in flight)
  // and the events that order it against the pass's stream
  hipStream_t ref_stream = nullptr;
  hipEvent_t ref_fork = nullptr, ref_qkv = nullptr, ref_attn = nullptr, ref_join = nullptr;
  char *static_scratch = nullptr;  // this device's copy of `scratch` (es_score_batch_static)
  float *rew = nullptr;  // raw rewards of a reference set (es_calibrate_offset)
  size_t rew_cap = 0;
  int *flag = nullptr;
  // per-call metadata: host assembly -> pinned staging -> one upload
  std::vector<uint8_t> meta_asm;
  char *meta_host = nullptr, *meta_dev = nullptr;
  size_t meta_cap = 0;
  hipEvent_t meta_ev = nullptr;
  bool meta_pending = false;
  std::vector<std::pair<void *, size_t>> allocs;
  int64_t device_bytes = 0;
  std::vector<int32_t> order_scratch;
  // profiling (es_profile_enable / es_profile_collect)
  struct Rec {
    int cls;
    hipEvent_t a, b;
    double flops, bytes;
  };
  uint32_t prof_mask = 0;
  std::vector<hipEvent_t> ev_pool;
  size_t ev_used = 0;
  std::vector<Rec> prof_recs;
};

namespace {

es_status dalloc(es_model *m, void **p, size_t bytes) {
  bytes = std::max<size_t>(bytes, 256);
  hipError_t e = hipMalloc(p, bytes);
  if (e != hipSuccess)
    return fail(ES_ERR_HIP, "hipMalloc(%zu) failed: %s", bytes, hipGetErrorString(e));
  m->allocs.emplace_back(*p, bytes);
  m->device_bytes += (int64_t)bytes;
  e = hipMemset(*p, 0, bytes);
  if (e != hipSuccess) return fail(ES_ERR_HIP, "hipMemset failed: %s", hipGetErrorString(e));
  // the fill may still be running on the null stream, which the internal
  // (non-blocking) streams do not wait for
  e = hipDeviceSynchronize();
  if (e != hipSuccess) return fail(ES_ERR_HIP, "hipDeviceSynchronize failed: %s", hipGetErrorString(e));
  return ES_OK;
}

// Free one dalloc'ed buffer (the device must be idle on it).
void dfree(es_model *m, void *p) {
  if (!p) return;
  for (size_t i = 0; i < m->allocs.size(); ++i) {
    if (m->allocs[i].first == p) {
      m->device_bytes -= (int64_t)m->allocs[i].second;
      m->allocs.erase(m->allocs.begin() + (std::ptrdiff_t)i);
      (void)hipFree(p);
      return;
    }
  }
}

void release(es_model *m) {
  if (!m) return;
  (void)hipDeviceSynchronize();
  for (auto &a : m->allocs) (void)hipFree(a.first);
  m->allocs.clear();
  if (m->meta_host) (void)hipHostFree(m->meta_host);
  if (m->meta_dev) (void)hipFree(m->meta_dev);
  if (m->rew) (void)hipFree(m->rew);
  if (m->meta_ev) (void)hipEventDestroy(m->meta_ev);
  if (m->fork_ev) (void)hipEventDestroy(m->fork_ev);
  for (hipEvent_t e : {m->ref_fork, m->ref_qkv, m->ref_attn, m->ref_join})
    if (e) (void)hipEventDestroy(e);
  if (m->ref_stream) (void)hipStreamDestroy(m->ref_stream);
  for (auto &w : m->ws) {
    if (w.stream) (void)hipStreamDestroy(w.stream);
    if (w.done) (void)hipEventDestroy(w.done);
  }
  for (hipEvent_t e : m->ev_pool) (void)hipEventDestroy(e);
  delete m;
}

// Upload a [rows, cols] tensor into a zero-filled [rows_alloc, ld] device matrix
// of element size `elem`, mapping source row r to destination row rmap(r) and
// source column c to destination column cmap(c).
template <typename RM, typename CM>
es_status upload_matrix(es_model *m, void **dst, const es::TensorView &t, int64_t rows_alloc,
                        int64_t ld, RM rmap, CM cmap) {
  const int elem = t.elem;
  // runs of source columns that stay contiguous after the column map
  struct Run { int64_t src, dst, len; };
  std::vector<Run> runs;
  for (int64_t c = 0; c < t.cols; ++c) {
    const int64_t dc = cmap(c);
    if (!runs.empty() && runs.back().src + runs.back().len == c &&
        runs.back().dst + runs.back().len == dc)
      ++runs.back().len;
    else
      runs.push_back({c, dc, 1});
  }
  std::vector<uint8_t> host((size_t)(rows_alloc * ld * elem), 0);
  const uint8_t *src = static_cast<const uint8_t *>(t.data);
  for (int64_t r = 0; r < t.rows; ++r) {
    const int64_t dr = rmap(r);
    for (const Run &u : runs)
      std::memcpy(&host[(size_t)((dr * ld + u.dst) * elem)], src + (r * t.cols + u.src) * elem,
                  (size_t)(u.len * elem));
  }
  es_status s = dalloc(m, dst, host.size());
  if (s != ES_OK) return s;
  HIP_TRY(hipMemcpy(*dst, host.data(), host.size(), hipMemcpyHostToDevice));
  return ES_OK;
}

es_status upload_vec(es_model *m, float **dst, const es::TensorView &t, int64_t n_alloc,
                     int64_t (*map)(int64_t, const es_model *) = nullptr) {
  std::vector<float> host((size_t)n_alloc, 0.f);
  const float *src = static_cast<const float *>(t.data);
  for (int64_t i = 0; i < t.cols; ++i) host[(size_t)(map ? map(i, m) : i)] = src[i];
  es_status s = dalloc(m, (void **)dst, host.size() * sizeof(float));
  if (s != ES_OK) return s;
  HIP_TRY(hipMemcpy(*dst, host.data(), host.size() * sizeof(float), hipMemcpyHostToDevice));
  return ES_OK;
}

// Row r of W_qkv (part p = r / H, head h, dim e) -> head-padded row.
int64_t qkv_row(int64_t r, const es_model *m) {
  const int64_t part = r / m->H, rem = r % m->H, h = rem / m->d, e = rem % m->d;
  return part * m->A * m->dp + h * m->dp + e;
}
int64_t ctx_col(int64_t c, const es_model *m) { return (c / m->d) * m->dp + c % m->d; }

double ms_since(const std::chrono::steady_clock::time_point &t0) {
  return std::chrono::duration<double, std::milli>(std::chrono::steady_clock::now() - t0).count();
}

// 4-byte words per sequence of the last-token refinement: its residual row
// and Q | K | V row (fp32), and its LayerNorm output, context and FFN middle
// rows (hi + lo bf16 pairs); sequences are counted in whole tiles of 32
// (refine_rows) since the split GEMMs read their operands tile by tile.
int64_t refine_floats(const es_model *m) {
  return m->refine_ok ? (int64_t)2 * m->H + m->Nqkv + m->Kc + m->Fp : 0;
}

int64_t refine_bytes(const es_model *m, int64_t n_seqs) {
  return ((n_seqs + 31) / 32 * 32) * refine_floats(m) * 4;
}

// Device bytes of all workspaces (fixed buffers or arenas).
int64_t work_bytes(const es_model *m) {
  int64_t b = 0;
  for (const auto &w : m->ws) {
    b += w.arena_cap;
    if (w.scale > 0) {
      const int act = m->bf16 ? 2 : 4;
      const int64_t T = round_up(w.scale * m->max_tokens, 256), S = w.scale * m->score_cap;
      b += T * (m->H * 8 + (int64_t)(m->Hp + m->Nqkv + m->Kc + m->Fp) * act) + S * (4 + act) +
           refine_bytes(m, (int64_t)w.scale * m->max_seqs);
    }
  }
  return b;
}

void free_fixed(es_model *m, es_model::Workspace &w) {
  if (w.arena) return;  // the tensor pointers are views into the arena
  for (void *p : {(void *)w.x, (void *)w.y, (void *)w.S, w.xb, w.qkv, w.ctx, w.hmid, w.Pb, (void *)w.ref})
    dfree(m, p);
  w.x = w.y = w.S = w.ref = nullptr;
  w.xb = w.qkv = w.ctx = w.hmid = w.Pb = nullptr;
  w.scale = 0;
}

void free_arena(es_model *m, es_model::Workspace &w) {
  if (!w.arena) return;
  dfree(m, w.arena);
  w.arena = nullptr;
  w.arena_cap = 0;
  w.x = w.y = w.S = w.ref = nullptr;
  w.xb = w.qkv = w.ctx = w.hmid = w.Pb = nullptr;
}

// Activation and score buffers for `scale` planned batches of up to
// max_tokens tokens each (fixed memory mode), zero-filled once so padding
// columns stay zero; a workspace that already holds buffers is resized.
es_status alloc_workspace(es_model *m, es_model::Workspace &w, int scale) {
  const auto t0 = std::chrono::steady_clock::now();
  free_arena(m, w);
  free_fixed(m, w);
  const int act = m->bf16 ? 2 : 4;
  const int64_t T = round_up(scale * m->max_tokens, 256);
  const int64_t S = scale * m->score_cap;
  es_status s;
  if ((s = dalloc(m, (void **)&w.x, T * m->H * 4)) != ES_OK) return s;
  if ((s = dalloc(m, (void **)&w.y, T * m->H * 4)) != ES_OK) return s;
  if ((s = dalloc(m, &w.xb, T * m->Hp * act)) != ES_OK) return s;
  if ((s = dalloc(m, &w.qkv, T * m->Nqkv * act)) != ES_OK) return s;
  if ((s = dalloc(m, &w.ctx, T * m->Kc * act)) != ES_OK) return s;
  if ((s = dalloc(m, &w.hmid, T * m->Fp * act)) != ES_OK) return s;
  if ((s = dalloc(m, (void **)&w.S, S * 4)) != ES_OK) return s;
  if ((s = dalloc(m, &w.Pb, S * act)) != ES_OK) return s;
  if (m->refine_ok &&
      (s = dalloc(m, (void **)&w.ref, refine_bytes(m, (int64_t)scale * m->max_seqs))) != ES_OK)
    return s;
  w.scale = scale;
  m->work_allocs += m->refine_ok ? 9 : 8;
  m->work_alloc_ms += ms_since(t0);
  m->peak_work = std::max(m->peak_work, work_bytes(m));
  return ES_OK;
}

// ---- length-aware workspace (TurboTransformers review, Proposed method: a
// sequence-length-aware allocator for variable-length inputs).  A pass's
// intermediates are sized from its own token count and score blocks, and
// placed in one arena per pass in flight by es_plan_arena's rule: tensors
// whose steps do not meet share addresses.  Steps (one layer repeats 2..9;
// x and xb carry across layers): 0 embedding, 1 pre-LN LayerNorm, 2 QKV GEMM,
// 3 attention (scores, softmax, P.V or fused), 4 last-row gather, 5
// attention-out GEMM, 6 its LayerNorm, 7 FFN1, 8 FFN2, 9 FFN LayerNorm,
// 10 head.  Bytes shared over time hold any bit pattern, so the padding
// columns of the K-padded GEMM inputs are written with zeros by their
// producers every time (LayerNorm / embedding: xb past H; FFN1 computes its
// zero padding columns past F; attention clears ctx past A dp).
enum { kTX, kTXb, kTQkv, kTCtx, kTY, kTHmid, kTS, kTP, kTRef, kTensors };
constexpr int64_t kArenaAlign = 4096;
constexpr int64_t kArenaChunk = (int64_t)16 << 20;

std::vector<es::Usage> pass_usage(const es_model *m, int64_t rows, int64_t score_elems,
                                  int64_t n_seqs) {
  const int64_t act = m->bf16 ? 2 : 4;
  std::vector<es::Usage> u(kTensors);
  u[kTX] = {rows * m->H * 4, 0, 10};
  u[kTXb] = {rows * m->Hp * act, 0, 10};
  u[kTQkv] = {rows * m->Nqkv * act, 2, 5};
  u[kTCtx] = {rows * m->Kc * act, 3, 5};
  u[kTY] = {rows * m->H * 4, 4, 9};
  u[kTHmid] = {rows * m->Fp * act, 7, 8};
  u[kTS] = {score_elems * 4, 3, 3};
  u[kTP] = {score_elems * act, 3, 3};
  u[kTRef] = {m->refine ? refine_bytes(m, n_seqs) : 0, 0, 10};  // the pass's refinement rows
  return u;
}

// Point w's tensors at a pass of n_tokens tokens (and score_elems score
// elements when the unfused attention runs).  Fixed mode: nothing to do.
// Length-aware: the arena grows (once queued work is done, with 1/8
// headroom, in 16 MiB steps) when this pass needs more, and at a call's first
// pass it shrinks to the previous call's largest need (plus 1/8, in 16 MiB
// steps) when it holds at least twice that.  Exact: a fresh arena of exactly
// this pass's need.
es_status bind_workspace(es_model *m, es_model::Workspace &w, int64_t n_tokens, int64_t score_elems,
                         int64_t n_seqs, hipStream_t st) {
  if (m->mem_mode == ES_MEM_FIXED) return ES_OK;
  const int64_t rows = std::max<int64_t>(round_up(n_tokens, 256), 256);
  std::vector<int64_t> off;
  const int64_t need = es::plan_arena(pass_usage(m, rows, score_elems, n_seqs), kArenaAlign, off);
  w.call_need = std::max(w.call_need, need);
  int64_t want = 0;
  if (m->mem_mode == ES_MEM_EXACT)
    want = need;
  else if (need > w.arena_cap)
    want = round_up(need + need / 8, kArenaChunk);
  else if (w.first_in_call && w.prev_call_need > 0) {
    const int64_t target = round_up(std::max(w.prev_call_need, need) * 9 / 8, kArenaChunk);
    if (2 * target <= w.arena_cap) want = target;
  }
  w.first_in_call = false;
  if (want > 0) {
    const auto t0 = std::chrono::steady_clock::now();
    // earlier passes (this lane's, or a previous call's on another stream)
    // may still use the old arena
    HIP_TRY(hipDeviceSynchronize());
    free_fixed(m, w);
    free_arena(m, w);
    es_status s = dalloc(m, (void **)&w.arena, (size_t)want);
    if (s != ES_OK) return s;
    w.arena_cap = want;
    m->work_allocs += 1;
    m->work_alloc_ms += ms_since(t0);
    m->peak_work = std::max(m->peak_work, work_bytes(m));
  }
  char *a = w.arena;
  w.x = reinterpret_cast<float *>(a + off[kTX]);
  w.xb = a + off[kTXb];
  w.qkv = a + off[kTQkv];
  w.ctx = a + off[kTCtx];
  w.y = reinterpret_cast<float *>(a + off[kTY]);
  w.hmid = a + off[kTHmid];
  w.S = reinterpret_cast<float *>(a + off[kTS]);
  w.Pb = a + off[kTP];
  w.ref = reinterpret_cast<float *>(a + off[kTRef]);
  return ES_OK;
}

// Start of a scoring call: each lane's shrink check looks at the last call.
void begin_call(es_model *m) {
  for (auto &w : m->ws) {
    if (w.call_need > 0) w.prev_call_need = w.call_need;
    w.call_need = 0;
    w.first_in_call = true;
  }
}

// Device address of `scratch` on `device`, looked up once per device (with
// that device current) and kept for the life of the process.
es_status static_scratch_of(int device, char **out) {
  static std::mutex mu;
  static std::vector<char *> addr;
  std::lock_guard<std::mutex> lock(mu);
  if (device < 0) return fail(ES_ERR_ARG, "device %d", device);
  if ((size_t)device >= addr.size()) addr.resize((size_t)device + 1, nullptr);
  if (!addr[device]) {
    int cur = 0;
    HIP_TRY(hipGetDevice(&cur));
    if (cur != device) HIP_TRY(hipSetDevice(device));
    void *p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != device) HIP_TRY(hipSetDevice(cur));
    if (e != hipSuccess || !p)
      return fail(ES_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d failed: %s", device,
                  hipGetErrorString(e));
    addr[device] = static_cast<char *>(p);
  }
  *out = addr[device];
  return ES_OK;
}

es_status build(const es::ParsedBlob &pb, int64_t max_tokens, int32_t max_seqs, es_model *m) {
  const es::BlobHeader &h = pb.h;
  m->L = (int)h.n_layers;
  m->H = (int)h.hidden;
  m->A = (int)h.n_heads;
  m->d = m->H / m->A;
  m->dp = pow2_at_least(m->d);
  m->F = (int)h.ffn;
  m->V = (int)h.vocab;
  m->P = (int)h.max_pos;
  m->pre_ln = h.pre_ln != 0;
  m->causal = h.causal != 0;
  m->bf16 = h.wdtype == 1;
  m->attn_mode = m->bf16 ? 1 : 0;
  static_assert(es::kLastMaxKeysHost >= es::kMaxPos, "the last-token attention holds every position");
  m->refine_ok = m->bf16 && m->pre_ln && h.hidden % 64 == 0 && h.ffn % 64 == 0;
  m->refine = m->refine_ok;
  m->eps = h.eps;
  m->offset = h.reward_offset;
  m->Hp = (int)round_up(m->H, 64);
  m->Nqkv = 3 * m->A * m->dp;
  m->Kc = (int)round_up((int64_t)m->A * m->dp, 64);
  m->Fp = (int)round_up(m->F, 64);
  m->max_tokens = max_tokens;
  m->max_seqs = max_seqs;
  m->Tcap = round_up(max_tokens, 256);
  const int64_t lmax = std::min<int64_t>(m->P, max_tokens);
  m->score_cap = (int64_t)m->A * max_tokens * es::score_ld((int)lmax);
  HIP_TRY(hipGetDevice(&m->device));

  es_status s;
  auto id = [](int64_t r) { return r; };
  // embeddings keep their natural [rows, H] layout
  if ((s = upload_matrix(m, &m->tok_emb, pb.tok_emb, m->V, m->H, id, id)) != ES_OK) return s;
  if ((s = upload_matrix(m, &m->pos_emb, pb.pos_emb, m->P, m->H, id, id)) != ES_OK) return s;
  if ((s = upload_vec(m, &m->norm_g, pb.norm_g, m->H)) != ES_OK) return s;
  if ((s = upload_vec(m, &m->norm_b, pb.norm_b, m->H)) != ES_OK) return s;
  if ((s = upload_vec(m, &m->head_w, pb.head_w, m->H)) != ES_OK) return s;
  if ((s = upload_vec(m, &m->head_b, pb.head_b, 1)) != ES_OK) return s;
  m->layers.assign(m->L, DevLayer{});
  const es_model *cm = m;
  for (int l = 0; l < m->L; ++l) {
    const es::LayerViews &L = pb.layers[l];
    DevLayer &D = m->layers[l];
    auto qrow = [cm](int64_t r) { return qkv_row(r, cm); };
    auto ccol = [cm](int64_t c) { return ctx_col(c, cm); };
    if ((s = upload_matrix(m, &D.w_qkv, L.w_qkv, round_up(m->Nqkv, 256), m->Hp, qrow, id)) != ES_OK) return s;
    if ((s = upload_vec(m, &D.b_qkv, L.b_qkv, m->Nqkv, qkv_row)) != ES_OK) return s;
    if ((s = upload_matrix(m, &D.w_o, L.w_o, round_up(m->H, 256), m->Kc, id, ccol)) != ES_OK) return s;
    if ((s = upload_vec(m, &D.b_o, L.b_o, m->H)) != ES_OK) return s;
    if ((s = upload_vec(m, &D.ln1_g, L.ln1_g, m->H)) != ES_OK) return s;
    if ((s = upload_vec(m, &D.ln1_b, L.ln1_b, m->H)) != ES_OK) return s;
    if ((s = upload_matrix(m, &D.w_1, L.w_1, round_up(m->F, 256), m->Hp, id, id)) != ES_OK) return s;
    if ((s = upload_vec(m, &D.b_1, L.b_1, m->Fp)) != ES_OK) return s;  // zero past F
    if ((s = upload_matrix(m, &D.w_2, L.w_2, round_up(m->H, 256), m->Fp, id, id)) != ES_OK) return s;
    if ((s = upload_vec(m, &D.b_2, L.b_2, m->H)) != ES_OK) return s;
    if ((s = upload_vec(m, &D.ln2_g, L.ln2_g, m->H)) != ES_OK) return s;
    if ((s = upload_vec(m, &D.ln2_b, L.ln2_b, m->H)) != ES_OK) return s;
  }
  m->ws.resize(1);
  if (m->mem_mode == ES_MEM_FIXED && (s = alloc_workspace(m, m->ws[0], 1)) != ES_OK) return s;
  if ((s = dalloc(m, (void **)&m->flag, 4)) != ES_OK) return s;
  HIP_TRY(hipEventCreateWithFlags(&m->meta_ev, hipEventDisableTiming));
  if (m->refine_ok) {  // default priority (every stream of the library)
    HIP_TRY(hipStreamCreateWithFlags(&m->ref_stream, hipStreamNonBlocking));
    for (hipEvent_t *e : {&m->ref_fork, &m->ref_qkv, &m->ref_attn, &m->ref_join})
      HIP_TRY(hipEventCreateWithFlags(e, hipEventDisableTiming));
  }
  if ((s = static_scratch_of(m->device, &m->static_scratch)) != ES_OK) return s;
  HIP_TRY(hipDeviceSynchronize());
  return ES_OK;
}

// ---- per-call metadata.  Every batch of a call gets offsets, score-block
// bases, attention work items and (optionally) id-source / reward-slot maps,
// assembled on the host, staged in pinned memory and uploaded in ONE copy.


// The layout parameters of a loaded model (layout.cpp builds the metadata).
es::LayoutParams layout_params(const es_model *m) {
  es::LayoutParams p;
  p.A = m->A;
  p.causal = m->causal;
  p.P = m->P;
  p.max_tokens = m->max_tokens;
  p.max_seqs = m->max_seqs;
  p.score_cap = m->score_cap;
  return p;
}

es_status add_batch(es_model *m, const int32_t *h_off, int32_t n, const int32_t *src,
                    const int32_t *dest, BatchLayout *L) {
  return es::add_batch(layout_params(m), m->meta_asm, m->order_scratch, h_off, n, src, dest, L);
}

// Stage m->meta_asm in pinned memory and enqueue its upload on `st`.
es_status upload_meta(es_model *m, hipStream_t st) {
  const size_t bytes = std::max<size_t>(m->meta_asm.size(), 16);
  // the previous call's upload must have left the staging buffer
  if (m->meta_pending) HIP_TRY(hipEventSynchronize(m->meta_ev));
  m->meta_pending = false;
  if (bytes > m->meta_cap) {
    const size_t cap = (size_t)round_up((int64_t)(bytes + bytes / 2), 4096);
    if (m->meta_dev) {
      HIP_TRY(hipStreamSynchronize(st));  // device copy may still be read by queued kernels
      HIP_TRY(hipDeviceSynchronize());
      HIP_TRY(hipFree(m->meta_dev));
      m->meta_dev = nullptr;
    }
    if (m->meta_host) {
      HIP_TRY(hipHostFree(m->meta_host));
      m->meta_host = nullptr;
    }
    m->meta_cap = 0;
    HIP_TRY(hipMalloc((void **)&m->meta_dev, cap));
    HIP_TRY(hipHostMalloc((void **)&m->meta_host, cap, hipHostMallocDefault));
    m->meta_cap = cap;
  }
  std::memcpy(m->meta_host, m->meta_asm.data(), m->meta_asm.size());
  HIP_TRY(hipMemcpyAsync(m->meta_dev, m->meta_host, bytes, hipMemcpyHostToDevice, st));
  HIP_TRY(hipEventRecord(m->meta_ev, st));
  m->meta_pending = true;
  return ES_OK;
}

// The last-token view of a layout, for the pruned last layer: `attn` keeps
// the packed offsets (and shared prompts) with one work item per sequence
// (its last query); `rows` lists the packed row of every last token; `tail`
// indexes the compacted rows 0..n-1 (offsets 0, 1, .., n) with the same
// reward slots.
struct LastView {
  es::Ragged attn, tail;
  const int32_t *rows = nullptr;
  int64_t pairs = 0;
};

es::Ragged ragged_of(const char *meta, const BatchLayout &L);

LastView last_view_of(const char *meta, const BatchLayout &L) {
  LastView v;
  v.attn = ragged_of(meta, L);
  v.attn.items = reinterpret_cast<const int32_t *>(meta + L.last_items);
  v.attn.n_items = L.n;
  v.attn.fused_items = v.attn.mw_items = nullptr;  // last queries: one tile each
  v.attn.n_fused_items = v.attn.n_mw_items = 0;
  v.attn.pfx_items = nullptr;
  v.attn.n_pfx_items = 0;
  v.rows = reinterpret_cast<const int32_t *>(meta + L.last_rows);
  v.tail = v.attn;
  v.tail.off = reinterpret_cast<const int32_t *>(meta + L.iota);
  v.tail.n_tokens = L.n;
  v.tail.pref = v.tail.plen = nullptr;
  v.pairs = L.last_pairs;
  return v;
}

es::Ragged ragged_of(const char *meta, const BatchLayout &L) {
  es::Ragged r;
  r.off = reinterpret_cast<const int32_t *>(meta + L.off);
  r.sbase = reinterpret_cast<const int64_t *>(meta + L.sbase);
  r.items = reinterpret_cast<const int32_t *>(meta + L.items);
  r.fused_items = reinterpret_cast<const int32_t *>(meta + L.fitems);
  r.mw_items = reinterpret_cast<const int32_t *>(meta + L.mitems);
  r.n_fused_items = L.n_fitems;
  r.n_mw_items = L.n_mitems;
  r.pfx_items = reinterpret_cast<const int32_t *>(meta + L.pitems);
  r.n_pfx_items = L.n_pitems;
  r.sm_items = reinterpret_cast<const int32_t *>(meta + L.sm_items);
  r.n_sm_items = L.n_sm_items;
  r.n_sm_narrow = L.n_sm_narrow;
  r.src = L.has_src ? reinterpret_cast<const int32_t *>(meta + L.src) : nullptr;
  r.dest = L.has_dest ? reinterpret_cast<const int32_t *>(meta + L.dest) : nullptr;
  r.pref = L.has_prefix ? reinterpret_cast<const int32_t *>(meta + L.pref) : nullptr;
  r.plen = L.has_prefix ? reinterpret_cast<const int32_t *>(meta + L.plen) : nullptr;
  r.n_seqs = L.n;
  r.n_items = L.n_items;
  r.max_len = L.max_len;
  r.n_tokens = L.n_tokens;
  return r;
}

// One batch given by host offsets: validate, stage, upload.
es_status prepare(es_model *m, const int32_t *h_off, int32_t n, hipStream_t st, es::Ragged *r,
                  int64_t *pairs, BatchLayout *layout = nullptr) {
  m->meta_asm.clear();
  BatchLayout L;
  es_status s = add_batch(m, h_off, n, nullptr, nullptr, &L);
  if (s != ES_OK) return s;
  if ((s = upload_meta(m, st)) != ES_OK) return s;
  *r = ragged_of(m->meta_dev, L);
  *pairs = L.pairs;
  if (layout) *layout = L;
  return ES_OK;
}

// ---- profiling: an event pair around each launch of a kernel class, with
// the algorithmic flops and HBM bytes of that launch (what the method must
// compute and move, no padding), aggregated by es_profile_collect.
struct Prof {
  es_model *m;
  hipStream_t st;
  int cls;
  hipEvent_t a = nullptr;
  Prof(es_model *m_, hipStream_t st_, int cls_) : m(m_), st(st_), cls(cls_) {
    if (m->prof_mask & (1u << cls)) a = next_event(m), (void)hipEventRecord(a, st);
  }
  void done(double flops, double bytes) {
    if (!a) return;
    hipEvent_t b = next_event(m);
    (void)hipEventRecord(b, st);
    m->prof_recs.push_back({cls, a, b, flops, bytes});
  }
  static hipEvent_t next_event(es_model *m) {
    if (m->ev_used == m->ev_pool.size()) {
      hipEvent_t e = nullptr;
      (void)hipEventCreate(&e);
      m->ev_pool.push_back(e);
    }
    return m->ev_pool[m->ev_used++];
  }
};

// Nreal (if >= 0): output columns the method computes when N includes
// padding columns (the FFN1 GEMM writes zeros there, for the next GEMM's K).
es_status gemm(es_model *m, int cls, const void *A, int lda, const void *W, const float *bias,
               const float *res, void *out, int ldc, int M, int N, int K, int Kreal, int epi,
               hipStream_t st, int Nreal = -1) {
  Prof p(m, st, cls);
  if (m->bf16)
    HIP_TRY(es::launch_gemm_bf16((const uint16_t *)A, lda, (const uint16_t *)W, bias, res, out, ldc,
                                 M, N, K,
                                 cls == ES_KC_FFN2 && epi == es::kEpiResidual ? es::kEpiResidualFfn : epi,
                                 st));
  else
    HIP_TRY(es::launch_gemm_f32((const float *)A, lda, (const float *)W, bias, res, (float *)out, ldc,
                                M, N, K, epi, st));
  const double a = m->bf16 ? 2.0 : 4.0, out_b = (epi == es::kEpiBias || epi == es::kEpiGelu) ? a : 4.0;
  const double Nr = Nreal >= 0 ? Nreal : N;
  p.done(2.0 * M * Nr * Kreal,
         (double)M * Kreal * a + Nr * Kreal * a + (double)M * Nr * out_b +
             (epi == es::kEpiResidual ? 4.0 * M * Nr : 0.0) + 4.0 * Nr);
  return ES_OK;
}

using Workspace = es_model::Workspace;

es_status attention_heads(es_model *m, Workspace &w, const es::Ragged &r, int64_t pairs, hipStream_t st);

// The heads write context columns [0, A dp); when Kc is larger the band
// [A dp, Kc) is cleared (the output GEMM reads K = Kc, and with
// length-aware memory those bytes may hold another tensor's bits).
es_status attention(es_model *m, Workspace &w, const es::Ragged &r, int64_t pairs, hipStream_t st) {
  es_status s = attention_heads(m, w, r, pairs, st);
  if (s != ES_OK || m->Kc == m->A * m->dp) return s;
  const int act = m->bf16 ? 2 : 4;
  HIP_TRY(es::launch_zero_cols(w.ctx, (int64_t)m->Kc * act, r.n_tokens, (int64_t)m->A * m->dp * act,
                               (int64_t)m->Kc * act, st));
  return ES_OK;
}

es_status attention_heads(es_model *m, Workspace &w, const es::Ragged &r, int64_t pairs, hipStream_t st) {
  const float scale = 1.0f / std::sqrt((float)m->d);
  const double a = m->bf16 ? 2.0 : 4.0, T = r.n_tokens, Hd = (double)m->H;
  if (m->bf16 && (m->attn_mode == 1 || r.plen)) {  // shared prompts: fused only
    Prof p(m, st, ES_KC_ATTN_FUSED);
    HIP_TRY(es::launch_attn_fused((const uint16_t *)w.qkv, m->Nqkv, m->A, m->dp, scale, m->causal, r,
                                  (uint16_t *)w.ctx, m->Kc, st));
    p.done(4.0 * m->d * pairs, 4.0 * T * Hd * a);  // Q, K, V read, ctx written
    return ES_OK;
  }
  {
    Prof p(m, st, ES_KC_SCORES);
    HIP_TRY(es::launch_scores(m->bf16, w.qkv, m->Nqkv, m->A, m->dp, scale, m->causal, r, w.S, st));
    p.done(2.0 * m->d * pairs, 2.0 * T * Hd * a + 4.0 * pairs);
  }
  {
    Prof p(m, st, ES_KC_SOFTMAX);
    HIP_TRY(es::launch_softmax(m->bf16, w.S, w.Pb, r, m->A, m->causal, st));
    p.done(4.0 * pairs, (4.0 + a) * pairs);
  }
  {
    Prof p(m, st, ES_KC_PV);
    HIP_TRY(es::launch_pv(m->bf16, w.Pb, w.qkv, m->Nqkv, m->A, m->dp, m->causal, r, w.ctx, m->Kc, st));
    p.done(2.0 * m->d * pairs, a * pairs + 2.0 * T * Hd * a);
  }
  return ES_OK;
}

// LayerNorm of x (of x + sub, a residual connection, when sub is non-NULL)
// into y (fp32, nullable) and the bf16 / fp32 GEMM input w.xb.
es_status layernorm(es_model *m, Workspace &w, const float *x, const float *g, const float *b, int T,
                    float *y, hipStream_t st, const float *sub = nullptr) {
  Prof p(m, st, ES_KC_LAYERNORM);
  HIP_TRY(es::launch_layernorm(m->bf16, x, sub, g, b, T, m->H, m->eps, y, w.xb, m->Hp, m->Hp, st));
  const double a = m->bf16 ? 2.0 : 4.0;
  p.done((sub ? 9.0 : 8.0) * T * m->H, (double)T * m->H * (4.0 + a + (y ? 4.0 : 0.0) + (sub ? 4.0 : 0.0)));
  return ES_OK;
}

// Copy each last-token row of the residual stream (x -> y rows 0..n-1) and
// of the attention context (ctx -> qkv rows 0..n-1, pitch Nqkv) for the
// pruned last layer; the full-size contents of both sources are dead after.
es_status gather_last(es_model *m, Workspace &w, const LastView &lv, hipStream_t st) {
  Prof p(m, st, ES_KC_GATHER);
  const int act = m->bf16 ? 2 : 4, n = lv.tail.n_seqs;
  HIP_TRY(es::launch_gather_rows(w.x, m->H * 4, w.y, m->H * 4, m->H * 4, w.ctx, m->Kc * act, w.qkv,
                                 m->Nqkv * act, m->Kc * act, lv.rows, n, st));
  p.done(0.0, 2.0 * n * (m->H * 4.0 + m->Kc * act));
  return ES_OK;
}

// ---- last-token refinement (pre-LN bf16 models).  The reward reads one
// row per sequence, and in bf16 most of its error is that row's own rounding
// (its LayerNorm outputs, context and FFN middle rounded to bf16 at every
// layer).  So beside the bulk pass the last row of each sequence is carried
// in fp32: its GEMMs take the fp32 activations as hi + lo bf16 pairs against
// the same bf16 weights, and its attention runs in fp32 over the bulk's K / V
// of the other positions and its own fp32 K / V.  Only the last rows change:
// every other row (and so every key and value) is the bulk pass's.
struct RefineRows {
  float *x, *q;           // residual, Q | K | V (fp32 rows)
  uint16_t *u, *c, *h;    // LayerNorm out, context, FFN middle (split-operand layout)
};

RefineRows refine_rows(const es_model *m, const Workspace &w, int n) {
  const int64_t n32 = (n + 31) / 32 * 32;
  RefineRows R;
  R.x = w.ref;
  R.q = R.x + n32 * m->H;
  R.u = reinterpret_cast<uint16_t *>(R.q + n32 * m->Nqkv);
  R.c = R.u + n32 * m->H * 2;
  R.h = R.c + n32 * m->Kc * 2;
  return R;
}

// The last-token rows of the residual stream after the embedding.
es_status refine_start(es_model *m, Workspace &w, const LastView &lv, hipStream_t st) {
  Prof p(m, st, ES_KC_REFINE);
  const int n = lv.tail.n_seqs;
  const RefineRows R = refine_rows(m, w, n);
  HIP_TRY(es::launch_gather_rows(w.x, m->H * 4, R.x, m->H * 4, m->H * 4, nullptr, 0, nullptr, 0, 0,
                                 lv.rows, n, st));
  p.done(0.0, 2.0 * n * m->H * 4.0);
  return ES_OK;
}

// One layer on the refined rows; w.qkv holds this layer's bulk Q | K | V.
// part 0: the refined rows' LayerNorm and Q | K | V; part 1: their
// attention over this layer's Q | K | V (w.qkv, still live) and the rest of
// the layer.  Part 1 runs right after the bulk attention, whose last key
// reads are then the likeliest still in the MALL.
es_status refine_layer(es_model *m, Workspace &w, const DevLayer &D, const LastView &lv,
                       hipStream_t st, int part, hipEvent_t attn_done = nullptr) {
  Prof p(m, st, ES_KC_REFINE);
  const int n = lv.tail.n_seqs, H = m->H;
  const RefineRows R = refine_rows(m, w, n);
  const uint16_t *Wq = (const uint16_t *)D.w_qkv, *Wo = (const uint16_t *)D.w_o;
  const uint16_t *W1 = (const uint16_t *)D.w_1, *W2 = (const uint16_t *)D.w_2;
  const double Hd = (double)m->A * m->d, F = m->F, pr = (double)lv.pairs;
  if (part == 0) {
    HIP_TRY(es::launch_layernorm_split(R.x, D.ln1_g, D.ln1_b, n, H, m->eps, R.u, st));
    HIP_TRY(es::launch_gemm_split(R.u, Wq, D.b_qkv, nullptr, R.q, nullptr, m->Nqkv, n, m->Nqkv, H,
                                  es::kEpiF32, st));
    p.done(2.0 * n * 3.0 * H * Hd * 2.0, 2.0 * 3.0 * H * Hd + 4.0 * n * (3.0 * H + 3.0 * Hd));
    return ES_OK;
  }
  HIP_TRY(es::launch_attn_last((const uint16_t *)w.qkv, m->Nqkv, R.q, m->Nqkv, m->A, m->dp,
                               1.0f / std::sqrt((float)m->d), lv.attn, R.c, m->Kc, st));
  if (attn_done) HIP_TRY(hipEventRecord(attn_done, st));  // the last read of w.qkv
  HIP_TRY(es::launch_gemm_split(R.c, Wo, D.b_o, R.x, R.x, nullptr, H, n, H, m->Kc, es::kEpiResidual, st));
  HIP_TRY(es::launch_layernorm_split(R.x, D.ln2_g, D.ln2_b, n, H, m->eps, R.u, st));
  HIP_TRY(es::launch_gemm_split(R.u, W1, D.b_1, nullptr, nullptr, R.h, 0, n, m->Fp, H, es::kEpiGelu, st));
  HIP_TRY(es::launch_gemm_split(R.h, W2, D.b_2, R.x, R.x, nullptr, H, n, H, m->Fp, es::kEpiResidual, st));
  // bytes: the layer's bf16 weights once, the bf16 K and V of every
  // (last query, key, head) once, and the fp32 rows each step reads and writes
  p.done(2.0 * n * (H * Hd + 2.0 * H * F) * 2.0 + 4.0 * m->d * pr,
         2.0 * (H * Hd + 2.0 * H * F) + 4.0 * m->d * pr + 4.0 * n * (7.0 * H + 5.0 * Hd + 2.0 * F));
  return ES_OK;
}

// Embedding and n_layers layers.  With `last` (scoring), the last layer runs
// its QKV GEMM on every token (all keys and values are needed) and everything
// after it on the last token of each sequence only -- the reward reads nothing
// else -- leaving the final states in x rows 0..n_seqs-1 (head: last->tail).
// Each row's arithmetic is unchanged (GEMMs, LayerNorm are per row; the last
// query sees the same key tiles in the same order), so rewards are bitwise
// those of the full last layer.
es_status forward(es_model *m, Workspace &w, const int32_t *d_ids, const es::Ragged &r,
                  int64_t pairs, int n_layers, hipStream_t st, const LastView *last = nullptr,
                  bool prune = true) {
  const int T = r.n_tokens, H = m->H, F = m->F, Hd = m->A * m->d;
  const double a = m->bf16 ? 2.0 : 4.0;
  const bool fused = m->bf16 && (m->attn_mode == 1 || r.plen);
  es_status s;
  {
    Prof p(m, st, ES_KC_EMBED);
    HIP_TRY(es::launch_embed(m->bf16, m->bf16, !m->pre_ln, d_ids, r, m->tok_emb, m->pos_emb, m->V, H,
                             m->norm_g, m->norm_b, m->eps, w.x, w.xb, m->Hp, m->flag, st));
    p.done(10.0 * T * H, (double)T * H * (2.0 * a + 4.0 + (m->pre_ln ? 0.0 : a)) + 4.0 * T);
  }
  const bool refine = last && m->refine;
  if (refine && (s = refine_start(m, w, *last, st)) != ES_OK) return s;
  // With one pass in flight the refinement runs on a stream of its own
  // (rs), beside the pass's compute-bound GEMMs: it touches only its own
  // rows (the arena region kTRef, live all pass) and reads the bulk Q | K | V
  // of the layer (w.qkv).  Its attention waits for the layer's QKV GEMM; the
  // bulk FFN1 GEMM -- the first step that may reuse the Q | K | V memory
  // (arena steps 7-8 against 2-5), and before the next layer's QKV GEMM --
  // waits for that attention; the pass's stream waits for the whole side
  // stream before the head reads the refined rows.  With more passes in
  // flight they fill each other's gaps, and more streams than the GPU's
  // hardware queues would serialise, so the refinement stays on the pass's
  // stream; so it does under the profiling hook, whose per-class times are
  // those of kernels running alone.
  const bool side = refine && m->lanes == 1 && m->ref_stream && m->prof_mask == 0;
  hipStream_t rs = side ? m->ref_stream : st;
  if (side) {
    HIP_TRY(hipEventRecord(m->ref_fork, st));  // the gathered rows
    HIP_TRY(hipStreamWaitEvent(rs, m->ref_fork, 0));
  }
  for (int l = 0; l < n_layers; ++l) {
    const DevLayer &D = m->layers[l];
    const bool tail = last && prune && l == n_layers - 1;
    if (!m->pre_ln) {
      if ((s = gemm(m, ES_KC_QKV, w.xb, m->Hp, D.w_qkv, D.b_qkv, nullptr, w.qkv, m->Nqkv, T,
                    m->Nqkv, m->Hp, H, es::kEpiBias, st)) != ES_OK) return s;
      if (!tail) {
        if ((s = attention(m, w, r, pairs, st)) != ES_OK) return s;
        if ((s = gemm(m, ES_KC_OPROJ, w.ctx, m->Kc, D.w_o, D.b_o, w.x, w.y, H, T, H, m->Kc, Hd,
                      es::kEpiResidual, st)) != ES_OK) return s;
        if ((s = layernorm(m, w, w.y, D.ln1_g, D.ln1_b, T, w.x, st)) != ES_OK) return s;
        if ((s = gemm(m, ES_KC_FFN1, w.xb, m->Hp, D.w_1, D.b_1, nullptr, w.hmid, m->Fp, T, m->Fp, m->Hp,
                      H, es::kEpiGelu, st, F)) != ES_OK) return s;
        // the residual joins in the LayerNorm: the GEMM's output tiles then
        // end without a read (its grid is often a single wave of tiles, whose
        // epilogues all hit HBM at once), and LayerNorm streams it instead
        if ((s = gemm(m, ES_KC_FFN2, w.hmid, m->Fp, D.w_2, D.b_2, nullptr, w.y, H, T, H, m->Fp, F,
                      es::kEpiF32, st)) != ES_OK) return s;
        if ((s = layernorm(m, w, w.x, D.ln2_g, D.ln2_b, T, w.x, st, w.y)) != ES_OK) return s;
      } else {
        const int n = last->tail.n_seqs;
        if ((s = attention(m, w, fused ? last->attn : r, fused ? last->pairs : pairs, st)) != ES_OK) return s;
        if ((s = gather_last(m, w, *last, st)) != ES_OK) return s;  // x -> y, ctx -> qkv
        if ((s = gemm(m, ES_KC_OPROJ, w.qkv, m->Nqkv, D.w_o, D.b_o, w.y, w.x, H, n, H, m->Kc, Hd,
                      es::kEpiResidual, st)) != ES_OK) return s;
        if ((s = layernorm(m, w, w.x, D.ln1_g, D.ln1_b, n, w.y, st)) != ES_OK) return s;
        if ((s = gemm(m, ES_KC_FFN1, w.xb, m->Hp, D.w_1, D.b_1, nullptr, w.hmid, m->Fp, n, m->Fp, m->Hp,
                      H, es::kEpiGelu, st, F)) != ES_OK) return s;
        if ((s = gemm(m, ES_KC_FFN2, w.hmid, m->Fp, D.w_2, D.b_2, w.y, w.x, H, n, H, m->Fp, F,
                      es::kEpiResidual, st)) != ES_OK) return s;
        if ((s = layernorm(m, w, w.x, D.ln2_g, D.ln2_b, n, w.x, st)) != ES_OK) return s;
      }
    } else {
      if ((s = layernorm(m, w, w.x, D.ln1_g, D.ln1_b, T, nullptr, st)) != ES_OK) return s;
      if ((s = gemm(m, ES_KC_QKV, w.xb, m->Hp, D.w_qkv, D.b_qkv, nullptr, w.qkv, m->Nqkv, T,
                    m->Nqkv, m->Hp, H, es::kEpiBias, st)) != ES_OK) return s;
      if (refine && (s = refine_layer(m, w, D, *last, rs, 0)) != ES_OK) return s;
      if (side) {  // the layer's bulk Q | K | V
        HIP_TRY(hipEventRecord(m->ref_qkv, st));
        HIP_TRY(hipStreamWaitEvent(rs, m->ref_qkv, 0));
      }
      if (side && !tail &&
          (s = refine_layer(m, w, D, *last, rs, 1, m->ref_attn)) != ES_OK) return s;
      if (!tail) {
        if ((s = attention(m, w, r, pairs, st)) != ES_OK) return s;
        // before anything of the bulk layer may reuse the Q | K | V memory
        if (refine && !side && (s = refine_layer(m, w, D, *last, st, 1)) != ES_OK) return s;
        if ((s = gemm(m, ES_KC_OPROJ, w.ctx, m->Kc, D.w_o, D.b_o, w.x, w.x, H, T, H, m->Kc, Hd,
                      es::kEpiResidual, st)) != ES_OK) return s;
        if ((s = layernorm(m, w, w.x, D.ln2_g, D.ln2_b, T, nullptr, st)) != ES_OK) return s;
        if (side) HIP_TRY(hipStreamWaitEvent(st, m->ref_attn, 0));  // w.qkv read by rs
        if ((s = gemm(m, ES_KC_FFN1, w.xb, m->Hp, D.w_1, D.b_1, nullptr, w.hmid, m->Fp, T, m->Fp, m->Hp,
                      H, es::kEpiGelu, st, F)) != ES_OK) return s;
        if ((s = gemm(m, ES_KC_FFN2, w.hmid, m->Fp, D.w_2, D.b_2, w.x, w.x, H, T, H, m->Fp, F,
                      es::kEpiResidual, st)) != ES_OK) return s;
      } else if (refine) {  // the refined rows carry the pruned last layer
        if ((s = refine_layer(m, w, D, *last, rs, 1)) != ES_OK) return s;
      } else {
        const int n = last->tail.n_seqs;
        if ((s = attention(m, w, fused ? last->attn : r, fused ? last->pairs : pairs, st)) != ES_OK) return s;
        if ((s = gather_last(m, w, *last, st)) != ES_OK) return s;  // x -> y, ctx -> qkv
        if ((s = gemm(m, ES_KC_OPROJ, w.qkv, m->Nqkv, D.w_o, D.b_o, w.y, w.y, H, n, H, m->Kc, Hd,
                      es::kEpiResidual, st)) != ES_OK) return s;
        if ((s = layernorm(m, w, w.y, D.ln2_g, D.ln2_b, n, nullptr, st)) != ES_OK) return s;
        if ((s = gemm(m, ES_KC_FFN1, w.xb, m->Hp, D.w_1, D.b_1, nullptr, w.hmid, m->Fp, n, m->Fp, m->Hp,
                      H, es::kEpiGelu, st, F)) != ES_OK) return s;
        if ((s = gemm(m, ES_KC_FFN2, w.hmid, m->Fp, D.w_2, D.b_2, w.y, w.x, H, n, H, m->Fp, F,
                      es::kEpiResidual, st)) != ES_OK) return s;
      }
    }
  }
  if (side) {  // the refined rows, before the head reads them
    HIP_TRY(hipEventRecord(m->ref_join, rs));
    HIP_TRY(hipStreamWaitEvent(st, m->ref_join, 0));
  }
  (void)a;
  return ES_OK;
}

es_status head(es_model *m, const float *x, const es::Ragged &r, float offset, float *rewards,
               hipStream_t st) {
  Prof p(m, st, ES_KC_HEAD);
  HIP_TRY(es::launch_head(m->pre_ln, x, m->H, r, m->norm_g, m->norm_b, m->eps, m->head_w,
                          m->head_b, offset, rewards, st));
  p.done(2.0 * r.n_seqs * m->H, 8.0 * r.n_seqs * m->H);
  return ES_OK;
}

es_status check_model(const es_model *m) {
  if (!m) return fail(ES_ERR_ARG, "model handle is NULL");
  return ES_OK;
}

}  // namespace

// ------------------------------------------------------------------ C ABI

extern "C" es_status es_load_weights_mem(const void *h_blob, int64_t nbytes, int64_t max_tokens,
                                         int32_t max_seqs, es_model **out) {
  if (!out) return fail(ES_ERR_ARG, "out is NULL");
  *out = nullptr;
  if (max_tokens < 1 || max_tokens > (int64_t)1 << 28)
    return fail(ES_ERR_ARG, "max_tokens=%" PRId64 " outside [1, 2^28]", max_tokens);
  if (max_seqs < 1 || max_seqs > (1 << 24)) return fail(ES_ERR_ARG, "max_seqs=%d outside [1, 2^24]", max_seqs);
  es::ParsedBlob pb;
  es_status s = es::parse_blob(h_blob, nbytes, &pb);
  if (s != ES_OK) return s;
  es_model *m = new es_model();
  s = build(pb, max_tokens, max_seqs, m);
  if (s != ES_OK) {
    release(m);
    return s;
  }
  *out = m;
  es::clear_error();
  return ES_OK;
}

extern "C" es_status es_load_weights(const char *blob_path, int64_t max_tokens, int32_t max_seqs,
                                     es_model **out) {
  if (!blob_path || !out) return fail(ES_ERR_ARG, "NULL path or out");
  std::ifstream f(blob_path, std::ios::binary | std::ios::ate);
  if (!f) return fail(ES_ERR_IO, "cannot open %s", blob_path);
  const std::streamsize size = f.tellg();
  f.seekg(0);
  std::vector<char> buf((size_t)size);
  if (!f.read(buf.data(), size)) return fail(ES_ERR_IO, "cannot read %s", blob_path);
  return es_load_weights_mem(buf.data(), (int64_t)size, max_tokens, max_seqs, out);
}

extern "C" void es_free(es_model *m) { release(m); }

extern "C" es_status es_model_info(const es_model *m, es_model_info_t *info) {
  if (!m || !info) return fail(ES_ERR_ARG, "NULL argument");
  info->n_layers = m->L;
  info->hidden = m->H;
  info->n_heads = m->A;
  info->head_dim = m->d;
  info->ffn = m->F;
  info->vocab = m->V;
  info->max_pos = m->P;
  info->pre_ln = m->pre_ln;
  info->causal = m->causal;
  info->bf16 = m->bf16;
  info->eps = m->eps;
  info->reward_offset = m->offset;
  info->max_tokens = m->max_tokens;
  info->max_seqs = m->max_seqs;
  info->device_bytes = m->device_bytes;
  return ES_OK;
}

// One pass of a laid-out batch: every layer, then the head.
es_status score_pass(es_model *m, Workspace &w, const int32_t *d_ids, const BatchLayout &L,
                     float *d_rewards, hipStream_t st, const char *meta = nullptr,
                     bool bound = false) {
  if (!meta) meta = m->meta_dev;
  const es::Ragged r = ragged_of(meta, L);
  const bool fused = m->bf16 && (m->attn_mode == 1 || L.has_prefix);
  es_status s;
  if (!bound && (s = bind_workspace(m, w, L.n_tokens, fused ? 0 : L.score_elems, L.n, st)) != ES_OK)
    return s;
  if ((m->prune || m->refine) && m->L > 0) {
    const LastView lv = last_view_of(meta, L);
    if ((s = forward(m, w, d_ids, r, L.pairs, m->L, st, &lv, m->prune)) != ES_OK) return s;
    return head(m, m->refine ? w.ref : w.x, lv.tail, m->offset, d_rewards, st);
  }
  if ((s = forward(m, w, d_ids, r, L.pairs, m->L, st)) != ES_OK) return s;
  return head(m, w.x, r, m->offset, d_rewards, st);
}

extern "C" es_status es_score_batch(es_model *m, const int32_t *d_token_ids, const int32_t *h_offsets,
                                    int32_t n_seqs, float *d_rewards, void *stream) {
  es_status s = check_model(m);
  if (s != ES_OK) return s;
  if (!d_token_ids || !d_rewards) return fail(ES_ERR_ARG, "NULL device pointer");
  hipStream_t st = static_cast<hipStream_t>(stream);
  es::Ragged r;
  int64_t pairs = 0;
  BatchLayout L;
  begin_call(m);
  if ((s = prepare(m, h_offsets, n_seqs, st, &r, &pairs, &L)) != ES_OK) return s;
  if ((s = score_pass(m, m->ws[0], d_token_ids, L, d_rewards, st)) != ES_OK) return s;
  es::clear_error();
  return ES_OK;
}

// es_score_batch with every intermediate in this device's `scratch`: the
// batch metadata first (aligned to kArenaAlign), then the pass's tensors at
// the offsets es_plan_arena gives their lifetimes (the length-aware layout).
// No device or pinned allocation: the metadata goes up by a copy from the
// host assembly buffer, and a batch whose need exceeds the array is refused.
extern "C" es_status es_score_batch_static(es_model *m, const int32_t *d_token_ids,
                                           const int32_t *h_offsets, int32_t n_seqs,
                                           float *d_rewards, void *stream) {
  es_status s = check_model(m);
  if (s != ES_OK) return s;
  if (!d_token_ids || !d_rewards) return fail(ES_ERR_ARG, "NULL device pointer");
  int dev = 0;
  HIP_TRY(hipGetDevice(&dev));
  if (dev != m->device)
    return fail(ES_ERR_ARG, "current device %d is not the model's device %d", dev, m->device);
  hipStream_t st = static_cast<hipStream_t>(stream);
  begin_call(m);
  m->meta_asm.clear();
  BatchLayout L;
  if ((s = add_batch(m, h_offsets, n_seqs, nullptr, nullptr, &L)) != ES_OK) return s;
  const bool fused = m->bf16 && m->attn_mode == 1;
  const int64_t rows = std::max<int64_t>(round_up(L.n_tokens, 256), 256);
  std::vector<int64_t> off;
  const int64_t need =
      es::plan_arena(pass_usage(m, rows, fused ? 0 : L.score_elems, L.n), kArenaAlign, off);
  const int64_t meta_bytes = round_up(std::max<int64_t>((int64_t)m->meta_asm.size(), 16), kArenaAlign);
  if (meta_bytes + need > ES_STATIC_SCRATCH_BYTES)
    return fail(ES_ERR_CAPACITY,
                "batch needs %" PRId64 " bytes of scratch (%" PRId64 " metadata + %" PRId64
                " tensors), above ES_STATIC_SCRATCH_BYTES=%lld",
                meta_bytes + need, meta_bytes, need, (long long)ES_STATIC_SCRATCH_BYTES);
  char *base = m->static_scratch;
  HIP_TRY(hipMemcpyAsync(base, m->meta_asm.data(), m->meta_asm.size(), hipMemcpyHostToDevice, st));
  Workspace w;
  char *a = base + meta_bytes;
  w.x = reinterpret_cast<float *>(a + off[kTX]);
  w.xb = a + off[kTXb];
  w.qkv = a + off[kTQkv];
  w.ctx = a + off[kTCtx];
  w.y = reinterpret_cast<float *>(a + off[kTY]);
  w.hmid = a + off[kTHmid];
  w.S = reinterpret_cast<float *>(a + off[kTS]);
  w.Pb = a + off[kTP];
  w.ref = reinterpret_cast<float *>(a + off[kTRef]);
  if ((s = score_pass(m, w, d_token_ids, L, d_rewards, st, base, true)) != ES_OK) return s;
  es::clear_error();
  return ES_OK;
}

extern "C" es_status es_score_requests(es_model *m, const int32_t *d_token_ids,
                                       const int32_t *h_lengths, int32_t n, int64_t batch_overhead,
                                       float *d_rewards, void *stream, es_stream_stats_t *stats) {
  es_status s = check_model(m);
  if (s != ES_OK) return s;
  if (!d_token_ids || !d_rewards || !h_lengths) return fail(ES_ERR_ARG, "NULL argument");
  if (n < 1) return fail(ES_ERR_ARG, "n=%d < 1", n);
  // a1 + a2 on the host (layout.cpp): plan the stream, pack groups of
  // planned batches into passes with id-source and reward-slot maps
  es::CallPlan plan;
  if ((s = es::build_stream(layout_params(m), h_lengths, n, batch_overhead, m->group, m->cost_table,
                            std::min(m->cost_max_batch, m->max_seqs), m->cost_max_len, m->meta_asm,
                            m->order_scratch, &plan)) != ES_OK)
    return s;
  const std::vector<BatchLayout> &layouts = plan.passes;
  const int32_t ng = (int32_t)layouts.size();
  hipStream_t st = static_cast<hipStream_t>(stream);
  if ((s = upload_meta(m, st)) != ES_OK) return s;
  // a3..a13: every group through the layers; the head scatters to request
  // order.  With k workspaces, group g runs on internal stream g % k, forked
  // from and joined back to the caller's stream.
  const int k = m->lanes;
  begin_call(m);
  if (k > 1) {
    HIP_TRY(hipEventRecord(m->fork_ev, st));
    for (int i = 0; i < k; ++i) HIP_TRY(hipStreamWaitEvent(m->ws[i].stream, m->fork_ev, 0));
  }
  for (int32_t g = 0; g < ng; ++g) {
    Workspace &w = m->ws[g % k];
    hipStream_t ls = k > 1 ? w.stream : st;
    if ((s = score_pass(m, w, d_token_ids, layouts[g], d_rewards, ls)) != ES_OK) return s;
  }
  if (k > 1) {
    for (int i = 0; i < k; ++i) {
      HIP_TRY(hipEventRecord(m->ws[i].done, m->ws[i].stream));
      HIP_TRY(hipStreamWaitEvent(st, m->ws[i].done, 0));
    }
  }
  if (stats) {
    stats->n_batches = plan.n_batches;
    stats->total_cost = plan.total_cost;
    stats->padded_tokens = plan.padded_tokens;
    stats->packed_tokens = plan.packed_tokens;
  }
  es::clear_error();
  return ES_OK;
}

extern "C" es_status es_score_best_of_n(es_model *m, const int32_t *d_token_ids,
                                        const int32_t *h_prompt_lengths, int32_t n_prompts,
                                        const int32_t *h_cand_lengths, const int32_t *h_cand_counts,
                                        int64_t batch_overhead, float *d_rewards, int32_t *d_best,
                                        void *stream, es_stream_stats_t *stats) {
  es_status s = check_model(m);
  if (s != ES_OK) return s;
  if (!d_token_ids || !d_rewards || !d_best || !h_prompt_lengths || !h_cand_lengths || !h_cand_counts)
    return fail(ES_ERR_ARG, "NULL argument");
  if (!m->causal || !m->bf16)
    return fail(ES_ERR_ARG, "shared-prompt scoring needs a causal bf16 model (a bidirectional "
                            "prompt's states depend on its continuation)");
  if (n_prompts < 1) return fail(ES_ERR_ARG, "n_prompts=%d < 1", n_prompts);
  // a1 + a2 on the host (layout.cpp): plan prompt groups, lay out each pass
  // as prompts followed by their candidates
  es::CallPlan plan;
  if ((s = es::build_best_of_n(layout_params(m), h_prompt_lengths, n_prompts, h_cand_lengths,
                               h_cand_counts, batch_overhead, m->group, m->meta_asm,
                               m->order_scratch, &plan)) != ES_OK)
    return s;
  const std::vector<BatchLayout> &layouts = plan.passes;
  const int32_t ng = (int32_t)layouts.size();
  const size_t cs_at = plan.cand_starts;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if ((s = upload_meta(m, st)) != ES_OK) return s;
  // a3..a13 per pass, passes in flight as in es_score_requests
  const int k = m->lanes;
  begin_call(m);
  if (k > 1) {
    HIP_TRY(hipEventRecord(m->fork_ev, st));
    for (int i = 0; i < k; ++i) HIP_TRY(hipStreamWaitEvent(m->ws[i].stream, m->fork_ev, 0));
  }
  for (int32_t gi = 0; gi < ng; ++gi) {
    Workspace &w = m->ws[gi % k];
    hipStream_t ls = k > 1 ? w.stream : st;
    if ((s = score_pass(m, w, d_token_ids, layouts[gi], d_rewards, ls)) != ES_OK) return s;
  }
  if (k > 1) {
    for (int i = 0; i < k; ++i) {
      HIP_TRY(hipEventRecord(m->ws[i].done, m->ws[i].stream));
      HIP_TRY(hipStreamWaitEvent(st, m->ws[i].done, 0));
    }
  }
  // selection: per prompt the best candidate, lowest index among equals
  HIP_TRY(es::launch_best_of_n(d_rewards, reinterpret_cast<const int32_t *>(m->meta_dev + cs_at),
                               n_prompts, d_best, st));
  if (stats) {
    stats->n_batches = plan.n_batches;
    stats->total_cost = plan.total_cost;
    stats->padded_tokens = plan.padded_tokens;
    stats->packed_tokens = plan.packed_tokens;
  }
  es::clear_error();
  return ES_OK;
}

extern "C" es_status es_forward_hidden(es_model *m, const int32_t *d_token_ids,
                                       const int32_t *h_offsets, int32_t n_seqs, int32_t n_layers,
                                       float *d_hidden, void *stream) {
  es_status s = check_model(m);
  if (s != ES_OK) return s;
  if (!d_token_ids || !d_hidden) return fail(ES_ERR_ARG, "NULL device pointer");
  if (n_layers < 0 || n_layers > m->L) return fail(ES_ERR_ARG, "n_layers=%d outside [0, %d]", n_layers, m->L);
  hipStream_t st = static_cast<hipStream_t>(stream);
  es::Ragged r;
  int64_t pairs = 0;
  BatchLayout L;
  begin_call(m);
  if ((s = prepare(m, h_offsets, n_seqs, st, &r, &pairs, &L)) != ES_OK) return s;
  const bool fused = m->bf16 && m->attn_mode == 1;
  if ((s = bind_workspace(m, m->ws[0], L.n_tokens, fused ? 0 : L.score_elems, 0, st)) != ES_OK) return s;
  if ((s = forward(m, m->ws[0], d_token_ids, r, pairs, n_layers, st)) != ES_OK) return s;
  HIP_TRY(hipMemcpyAsync(d_hidden, m->ws[0].x, (size_t)r.n_tokens * m->H * 4, hipMemcpyDeviceToDevice, st));
  return ES_OK;
}

extern "C" es_status es_set_concurrency(es_model *m, int32_t batches_in_flight) {
  if (!m) return fail(ES_ERR_ARG, "model handle is NULL");
  if (batches_in_flight < 1 || batches_in_flight > 4)
    return fail(ES_ERR_ARG, "batches_in_flight=%d outside [1, 4]", batches_in_flight);
  HIP_TRY(hipDeviceSynchronize());
  if (!m->fork_ev) HIP_TRY(hipEventCreateWithFlags(&m->fork_ev, hipEventDisableTiming));
  while ((int)m->ws.size() < batches_in_flight) m->ws.emplace_back();
  for (int i = 0; i < batches_in_flight; ++i) {
    es_model::Workspace &w = m->ws[i];
    if (m->mem_mode == ES_MEM_FIXED && w.scale < m->group) {
      es_status s = alloc_workspace(m, w, m->group);
      if (s != ES_OK) return s;
    }
    if (!w.stream) HIP_TRY(hipStreamCreateWithFlags(&w.stream, hipStreamNonBlocking));
    if (!w.done) HIP_TRY(hipEventCreateWithFlags(&w.done, hipEventDisableTiming));
  }
  m->lanes = batches_in_flight;  // extra workspaces stay allocated until es_free
  return ES_OK;
}

extern "C" es_status es_set_batch_grouping(es_model *m, int32_t batches_per_pass) {
  if (!m) return fail(ES_ERR_ARG, "model handle is NULL");
  if (batches_per_pass < 1 || batches_per_pass > 8)
    return fail(ES_ERR_ARG, "batches_per_pass=%d outside [1, 8]", batches_per_pass);
  HIP_TRY(hipDeviceSynchronize());
  m->group = batches_per_pass;
  for (int i = 0; i < m->lanes; ++i) {
    es_model::Workspace &w = m->ws[i];
    if (m->mem_mode == ES_MEM_FIXED && w.scale < m->group) {
      es_status s = alloc_workspace(m, w, m->group);
      if (s != ES_OK) return s;
    }
  }
  return ES_OK;
}

extern "C" es_status es_set_cost_table(es_model *m, const int64_t *cost_table, int32_t max_batch,
                                       int32_t max_len) {
  if (!m) return fail(ES_ERR_ARG, "model handle is NULL");
  if (!cost_table) {
    m->cost_table.clear();
    m->cost_max_batch = m->cost_max_len = 0;
    return ES_OK;
  }
  if (max_len < m->P) return fail(ES_ERR_ARG, "cost table max_len=%d below max_pos=%d", max_len, m->P);
  // the planner's own checks of the table (entries, monotone rows, size)
  int32_t start0 = 0, nb = 0;
  int64_t cost = 0;
  es_status s = es_plan_batches_measured(nullptr, 0, m->max_tokens, cost_table, max_batch, max_len,
                                         nullptr, &start0, &nb, &cost);
  if (s != ES_OK) return s;
  m->cost_table.assign(cost_table, cost_table + (size_t)max_batch * max_len);
  m->cost_max_batch = max_batch;
  m->cost_max_len = max_len;
  return ES_OK;
}

extern "C" es_status es_set_memory_mode(es_model *m, int32_t mode) {
  if (!m) return fail(ES_ERR_ARG, "model handle is NULL");
  if (mode != ES_MEM_FIXED && mode != ES_MEM_LENGTH_AWARE && mode != ES_MEM_EXACT)
    return fail(ES_ERR_ARG, "memory mode %d is not ES_MEM_FIXED, ES_MEM_LENGTH_AWARE or ES_MEM_EXACT", mode);
  HIP_TRY(hipDeviceSynchronize());
  m->mem_mode = mode;
  for (int i = 0; i < (int)m->ws.size(); ++i) {
    es_model::Workspace &w = m->ws[i];
    free_arena(m, w);
    free_fixed(m, w);
    w.call_need = w.prev_call_need = 0;
    if (mode == ES_MEM_FIXED && i < m->lanes) {
      es_status s = alloc_workspace(m, w, m->group);
      if (s != ES_OK) return s;
    }
  }
  return ES_OK;
}

extern "C" es_status es_memory_stats(es_model *m, es_memory_stats_t *out, int32_t reset) {
  if (!m || !out) return fail(ES_ERR_ARG, "NULL argument");
  out->mode = m->mem_mode;
  out->device_bytes = m->device_bytes;
  out->work_bytes = work_bytes(m);
  out->peak_work_bytes = std::max(m->peak_work, out->work_bytes);
  out->allocs = m->work_allocs;
  out->alloc_ms = m->work_alloc_ms;
  if (reset) {
    m->work_allocs = 0;
    m->work_alloc_ms = 0.0;
    m->peak_work = out->work_bytes;
  }
  return ES_OK;
}

extern "C" es_status es_set_pruning(es_model *m, int32_t enabled) {
  if (!m) return fail(ES_ERR_ARG, "model handle is NULL");
  if (enabled != 0 && enabled != 1) return fail(ES_ERR_ARG, "enabled=%d (0 or 1)", enabled);
  m->prune = enabled != 0;
  return ES_OK;
}

extern "C" es_status es_set_refinement(es_model *m, int32_t enabled) {
  if (!m) return fail(ES_ERR_ARG, "model handle is NULL");
  if (enabled != 0 && enabled != 1) return fail(ES_ERR_ARG, "enabled=%d (0 or 1)", enabled);
  if (enabled && !m->refine_ok)
    return fail(ES_ERR_ARG, "the last-token refinement needs a pre-LN bf16 model with hidden and FFN "
                            "widths multiples of 64");
  m->refine = enabled != 0;
  return ES_OK;
}

extern "C" es_status es_get_refinement(const es_model *m, int32_t *enabled) {
  if (!m || !enabled) return fail(ES_ERR_ARG, "NULL argument");
  *enabled = m->refine ? 1 : 0;
  return ES_OK;
}

extern "C" es_status es_set_attention(es_model *m, int32_t mode) {
  if (!m) return fail(ES_ERR_ARG, "model handle is NULL");
  if (mode != 0 && mode != 1) return fail(ES_ERR_ARG, "attention mode %d (0 unfused, 1 fused)", mode);
  if (mode == 1 && !m->bf16) return fail(ES_ERR_ARG, "fused attention needs a bf16 model");
  m->attn_mode = mode;
  return ES_OK;
}

extern "C" es_status es_set_reward_offset(es_model *m, float offset) {
  if (!m) return fail(ES_ERR_ARG, "model handle is NULL");
  if (!std::isfinite(offset)) return fail(ES_ERR_ARG, "offset is not finite");
  m->offset = offset;
  return ES_OK;
}

extern "C" es_status es_get_reward_offset(const es_model *m, float *offset) {
  if (!m || !offset) return fail(ES_ERR_ARG, "NULL argument");
  *offset = m->offset;
  return ES_OK;
}

extern "C" es_status es_calibrate_offset(es_model *m, const int32_t *d_token_ids,
                                         const int32_t *h_offsets, int32_t n_ref, void *stream,
                                         float *offset_out) {
  es_status s = check_model(m);
  if (s != ES_OK) return s;
  if (!offset_out || !d_token_ids || !h_offsets) return fail(ES_ERR_ARG, "NULL argument");
  if (n_ref < 1) return fail(ES_ERR_ARG, "n_ref=%d < 1", n_ref);
  if (h_offsets[0] != 0) return fail(ES_ERR_ARG, "offsets[0]=%d, must be 0", h_offsets[0]);
  std::vector<int32_t> lens((size_t)n_ref);
  for (int32_t i = 0; i < n_ref; ++i) {
    lens[i] = h_offsets[i + 1] - h_offsets[i];
    if (lens[i] < 1) return fail(ES_ERR_ARG, "offsets not strictly increasing at %d", i);
  }
  // raw rewards of the whole reference set through the planned-stream path
  // (any size; batch composition does not change a sequence's reward)
  if ((size_t)n_ref > m->rew_cap) {
    HIP_TRY(hipDeviceSynchronize());
    if (m->rew) HIP_TRY(hipFree(m->rew));
    m->rew = nullptr;
    m->rew_cap = 0;
    HIP_TRY(hipMalloc((void **)&m->rew, (size_t)n_ref * 4));
    m->rew_cap = (size_t)n_ref;
  }
  const float saved = m->offset;
  m->offset = 0.0f;
  s = es_score_requests(m, d_token_ids, lens.data(), n_ref, 1024, m->rew, stream, nullptr);
  m->offset = saved;
  if (s != ES_OK) return s;
  hipStream_t st = static_cast<hipStream_t>(stream);
  std::vector<float> raw((size_t)n_ref);
  HIP_TRY(hipMemcpyAsync(raw.data(), m->rew, raw.size() * 4, hipMemcpyDeviceToHost, st));
  HIP_TRY(hipStreamSynchronize(st));
  double acc = 0.0;
  for (float v : raw) acc += v;
  *offset_out = (float)(-(acc / n_ref));
  return ES_OK;
}

extern "C" es_status es_check_device_errors(es_model *m, void *stream) {
  es_status s = check_model(m);
  if (s != ES_OK) return s;
  hipStream_t st = static_cast<hipStream_t>(stream);
  int flag = 0;
  HIP_TRY(hipMemcpyAsync(&flag, m->flag, 4, hipMemcpyDeviceToHost, st));
  HIP_TRY(hipStreamSynchronize(st));
  if (flag) {
    HIP_TRY(hipMemsetAsync(m->flag, 0, 4, st));
    HIP_TRY(hipStreamSynchronize(st));
    return fail(ES_ERR_DEVICE_FLAG, "a token id outside [0, %d) was seen (row 0 used instead)", m->V);
  }
  return ES_OK;
}

// ------------------------------------------------------------------ profiling

extern "C" es_status es_profile_enable(es_model *m, uint32_t class_mask) {
  if (!m) return fail(ES_ERR_ARG, "model handle is NULL");
  m->prof_mask = class_mask & ((1u << ES_KC_COUNT) - 1);
  m->prof_recs.clear();
  m->ev_used = 0;
  return ES_OK;
}

extern "C" es_status es_profile_collect(es_model *m, es_kernel_stat_t *out) {
  if (!m || !out) return fail(ES_ERR_ARG, "NULL argument");
  for (int c = 0; c < ES_KC_COUNT; ++c) out[c] = es_kernel_stat_t{c, 0, 0.0, 0.0, 0.0};
  if (!m->prof_recs.empty()) HIP_TRY(hipEventSynchronize(m->prof_recs.back().b));
  for (const auto &rec : m->prof_recs) {
    float ms = 0.f;
    HIP_TRY(hipEventElapsedTime(&ms, rec.a, rec.b));
    es_kernel_stat_t &o = out[rec.cls];
    o.launches += 1;
    o.total_ms += ms;
    o.flops += rec.flops;
    o.bytes += rec.bytes;
  }
  m->prof_recs.clear();
  m->ev_used = 0;
  return ES_OK;
}

extern "C" const char *es_kernel_class_name(int32_t cls) {
  static const char *names[ES_KC_COUNT] = {"embed", "qkv_gemm", "scores", "softmax", "pv",
                                           "oproj_gemm", "layernorm", "ffn1_gemm", "ffn2_gemm",
                                           "head", "attn_fused", "gather", "refine"};
  return (cls >= 0 && cls < ES_KC_COUNT) ? names[cls] : "";
}
