// Row kernels: embedding (+LN), LayerNorm, ragged Softmax, reward head.
//
// TurboTransformers review (Proposed method): Softmax and LayerNorm are the
// hot spots besides the GEMMs and are computed as parallel per-row ("batch")
// reductions.  On gfx950 each row (or group of short rows) is owned by one
// 64-lane wavefront: coalesced 16-byte loads straight into registers, one
// pass over HBM in and out, reductions by butterfly shuffles inside the
// wavefront, no barriers.
#include <algorithm>

#include "device.h"
#include "kernels.h"

namespace es {

namespace {

constexpr int kRowsPerBlock = 4;  // one row per wavefront, 4 wavefronts per block

__device__ __forceinline__ float4 load4(const float *p) { return *reinterpret_cast<const float4 *>(p); }
__device__ __forceinline__ float4 load4(const uint16_t *p) {
  const uint2 u = *reinterpret_cast<const uint2 *>(p);
  return make_float4(bf2f(u.x & 0xffff), bf2f(u.x >> 16), bf2f(u.y & 0xffff), bf2f(u.y >> 16));
}
__device__ __forceinline__ void store4(float *p, float4 v) { *reinterpret_cast<float4 *>(p) = v; }
__device__ __forceinline__ void store4(uint16_t *p, float4 v) {
  uint2 u;
  u.x = f2bf2(v.x, v.y);
  u.y = f2bf2(v.z, v.w);
  *reinterpret_cast<uint2 *>(p) = u;
}

// LayerNorm of one row held as NC float4 chunks per lane (chunk c4 = lane + 64 j).
// Two passes over registers: mean, then the biased variance of (x - mean).
// Gains and shifts are loaded before the reductions so their latency overlaps.
// The affine parameters of the columns a lane owns (unconditional loads at
// in-bounds chunks, so they can be issued together with the row's own).
template <int NC>
__device__ __forceinline__ void ln_load_affine(float4 (&gg)[NC], float4 (&bb)[NC], int lane, int c4n,
                                               const float *__restrict__ g,
                                               const float *__restrict__ b) {
#pragma unroll
  for (int j = 0; j < NC; ++j) {
    const int c4 = min(lane + kWave * j, c4n - 1);
    gg[j] = load4(g + 4 * c4);
    bb[j] = load4(b + 4 * c4);
  }
}

template <int NC>
__device__ __forceinline__ void ln_apply(float4 (&v)[NC], const float4 (&gg)[NC],
                                         const float4 (&bb)[NC], int lane, int c4n, int cols,
                                         float eps) {
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < NC; ++j)
    if (lane + kWave * j < c4n) s += (v[j].x + v[j].y) + (v[j].z + v[j].w);
  const float mean = wave_sum(s) / (float)cols;
  float s2 = 0.f;
#pragma unroll
  for (int j = 0; j < NC; ++j) {
    if (lane + kWave * j < c4n) {
      const float a = v[j].x - mean, b2 = v[j].y - mean, c = v[j].z - mean, d = v[j].w - mean;
      s2 += (a * a + b2 * b2) + (c * c + d * d);
    }
  }
  const float var = wave_sum(s2) / (float)cols;
  const float rstd = 1.0f / sqrtf(var + eps);
#pragma unroll
  for (int j = 0; j < NC; ++j) {
    const int c4 = lane + kWave * j;
    if (c4 < c4n) {
      v[j].x = (v[j].x - mean) * rstd * gg[j].x + bb[j].x;
      v[j].y = (v[j].y - mean) * rstd * gg[j].y + bb[j].y;
      v[j].z = (v[j].z - mean) * rstd * gg[j].z + bb[j].z;
      v[j].w = (v[j].w - mean) * rstd * gg[j].w + bb[j].w;
    }
  }
}

template <int NC>
__device__ __forceinline__ void ln_row(float4 (&v)[NC], int lane, int c4n, int cols,
                                       const float *__restrict__ g, const float *__restrict__ b,
                                       float eps) {
  float4 gg[NC], bb[NC];
  ln_load_affine<NC>(gg, bb, lane, c4n, g, b);
  ln_apply<NC>(v, gg, bb, lane, c4n, cols, eps);
}

// With ADD, the row is x + sub (a residual connection followed by its
// LayerNorm); y may alias x or sub: a wavefront reads its whole row before
// it writes any of it, and no other wavefront touches that row.  A
// wavefront takes R consecutive rows: the affine parameters are loaded once
// for all of them (per row, at 2048 columns, they were 16 KB of L2 reads
// beside the row's 8 KB from HBM), and the next row's loads are in flight
// while the current row is reduced and stored.
template <int NC, typename OutB, bool ADD, int R>
__global__ __launch_bounds__(256) void layernorm_kernel(const float *x, const float *sub,
                                                        const float *__restrict__ g,
                                                        const float *__restrict__ b, int64_t rows,
                                                        int cols, float eps, float *y, OutB *yb,
                                                        int ldb, int padc4) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t r0 = ((int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6)) * R;
  if (r0 >= rows) return;
  const int c4n = cols >> 2;
  // every load is issued before any is used, at an in-bounds chunk (lanes
  // past the row end re-read its last chunk and are zeroed below) and an
  // in-bounds row (the row after the last is the last again, never stored):
  // loads under a per-chunk branch made the compiler wait for each chunk's
  // pair before issuing the next, one memory round trip per chunk
  constexpr int NS = R > 1 ? 2 : 1;  // register sets: the current row and the next
  float4 v[NS][NC], u[NS][NC], gg[NC], bb[NC];
  auto load_row = [&](int set, int64_t row) {
#pragma unroll
    for (int j = 0; j < NC; ++j) {
      const int c4 = min(lane + kWave * j, c4n - 1);
      v[set][j] = load4(x + row * cols + 4 * c4);
      if (ADD) u[set][j] = load4(sub + row * cols + 4 * c4);
    }
  };
  load_row(0, r0);
  ln_load_affine<NC>(gg, bb, lane, c4n, g, b);
#pragma unroll
  for (int i = 0; i < R; ++i) {
    const int cur = i % NS;
    const int64_t row = r0 + i;
    if (i + 1 < R) load_row((i + 1) % NS, min(row + 1, rows - 1));
    if (row >= rows) break;  // uniform over the wavefront
    float4(&w)[NC] = v[cur];
#pragma unroll
    for (int j = 0; j < NC; ++j) {  // selects, no branches
      const bool in = lane + kWave * j < c4n;
      if (ADD) {
        w[j].x += u[cur][j].x; w[j].y += u[cur][j].y; w[j].z += u[cur][j].z; w[j].w += u[cur][j].w;
      }
      w[j].x = in ? w[j].x : 0.f;
      w[j].y = in ? w[j].y : 0.f;
      w[j].z = in ? w[j].z : 0.f;
      w[j].w = in ? w[j].w : 0.f;
    }
    ln_apply<NC>(w, gg, bb, lane, c4n, cols, eps);
#pragma unroll
    for (int j = 0; j < NC; ++j) {
      const int c4 = lane + kWave * j;
      if (c4 < c4n) {
        if (y) store4(y + row * cols + 4 * c4, w[j]);
        if (yb) store4(yb + row * ldb + 4 * c4, w[j]);
      } else if (yb && c4 < padc4) {  // zero padding columns of the GEMM input
        store4(yb + row * ldb + 4 * c4, make_float4(0.f, 0.f, 0.f, 0.f));
      }
    }
  }
}

// Zero `words` 4-byte words at the start of each of `rows` rows (stride ld
// words): the padding band of a K-padded GEMM operand.  One wavefront per row.
__global__ __launch_bounds__(256) void zero_cols_kernel(char *base, int64_t ld, int rows, int words) {
  const int lane = threadIdx.x & (kWave - 1);
  const int row = blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  if (row >= rows) return;
  uint32_t *p = reinterpret_cast<uint32_t *>(base) + (int64_t)row * ld;
  for (int i = lane; i < words; i += kWave) p[i] = 0u;
}

// Token t of the packed batch belongs to sequence s; its id is read at
// src[s] + position, so a batch can be gathered straight out of a request
// stream kept in arrival order (the packing step costs no extra copy).
template <int NC, typename W, bool LN, typename OutB>
__global__ __launch_bounds__(256) void embed_kernel(const int32_t *__restrict__ ids,
                                                    const int32_t *__restrict__ off,
                                                    const int32_t *__restrict__ src,
                                                    const int32_t *__restrict__ plen, int n_seqs,
                                                    int T, const W *__restrict__ tok,
                                                    const W *__restrict__ pos, int vocab, int H,
                                                    const float *__restrict__ g,
                                                    const float *__restrict__ b, float eps,
                                                    float *__restrict__ x, OutB *__restrict__ xb,
                                                    int ldb, int padc4, int *flag) {
  const int lane = threadIdx.x & (kWave - 1);
  const int t = blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  if (t >= T) return;
  const int s = seq_of_token(off, n_seqs, t);
  const int j = t - off[s];                  // index within the sequence's own tokens
  const int p = j + (plen ? plen[s] : 0);    // position: restarts at 0, after a shared prompt
  int id = ids[(src ? src[s] : off[s]) + j];
  if (id < 0 || id >= vocab) {
    if (lane == 0) atomicOr(flag, 1);
    id = 0;
  }
  const int c4n = H >> 2;
  const W *tr = tok + (int64_t)id * H;
  const W *pr = pos + (int64_t)p * H;
  // all loads issued before any is used, at in-bounds chunks (as in the
  // LayerNorm kernel): lanes past the row end are zeroed by a select
  float4 v[NC], c[NC], gg[NC], bb[NC];
#pragma unroll
  for (int j = 0; j < NC; ++j) {
    const int c4 = min(lane + kWave * j, c4n - 1);
    v[j] = load4(tr + 4 * c4);
    c[j] = load4(pr + 4 * c4);
  }
  if (LN) ln_load_affine<NC>(gg, bb, lane, c4n, g, b);
#pragma unroll
  for (int j = 0; j < NC; ++j) {
    const bool in = lane + kWave * j < c4n;
    v[j].x = in ? v[j].x + c[j].x : 0.f;
    v[j].y = in ? v[j].y + c[j].y : 0.f;
    v[j].z = in ? v[j].z + c[j].z : 0.f;
    v[j].w = in ? v[j].w + c[j].w : 0.f;
  }
  if (LN) ln_apply<NC>(v, gg, bb, lane, c4n, H, eps);
#pragma unroll
  for (int j = 0; j < NC; ++j) {
    const int c4 = lane + kWave * j;
    if (c4 < c4n) {
      store4(x + (int64_t)t * H + 4 * c4, v[j]);
      if (LN) store4(xb + (int64_t)t * ldb + 4 * c4, v[j]);
    } else if (LN && c4 < padc4) {  // zero padding columns of the GEMM input
      store4(xb + (int64_t)t * ldb + 4 * c4, make_float4(0.f, 0.f, 0.f, 0.f));
    }
  }
}

constexpr float kLog2e = 1.44269504088896340736f;

// Eight probabilities (chunk of a row) to P: one 16-byte store of bf16
// (round to nearest even), or two float4 for an fp32 P.
__device__ __forceinline__ void store8(uint16_t *p, const float (&o)[8]) {
  *reinterpret_cast<uint4 *>(p) =
      make_uint4(f2bf2(o[0], o[1]), f2bf2(o[2], o[3]), f2bf2(o[4], o[5]), f2bf2(o[6], o[7]));
}
__device__ __forceinline__ void store8(float *p, const float (&o)[8]) {
  *reinterpret_cast<float4 *>(p) = make_float4(o[0], o[1], o[2], o[3]);
  *reinterpret_cast<float4 *>(p + 4) = make_float4(o[4], o[5], o[6], o[7]);
}

// Softmax over the ragged score rows (TurboTransformers review, Proposed
// method: Softmax as a parallel batch reduction over rows).  One item covers
// a run of rows of one sequence's [A * n, ld] score block whose rows need the
// same lane count G (softmax_item): G lanes own a row, each lane eight
// consecutive scores per chunk, read as two float4 straight into registers
// (branch-free: addresses clamped into the row, values past its end masked
// to -inf); only the chunks the item's longest row needs are touched.  The
// block walks its rows in passes of 256 / G rows (4 wavefronts) with the
// next pass's loads in flight while the current pass reduces, so a block
// keeps memory busy through its whole run instead of one round trip per
// pass.  Max and sum reduce by butterfly shuffles within the G-lane group
// (G = 128: within each of the row's two wavefronts, then across the pair
// through LDS);
// each chunk goes out as one 16-byte store, with zeros past the row's last
// score up to the next multiple of 8 (inside the row's allocated length; no
// reader looks there).  Rows are addressed through score_row_off, so causal
// blocks are read and written as their packed lower triangles.
template <int NJ>
__device__ __forceinline__ void softmax_load(const float *__restrict__ S, int64_t ro, int m, int c0,
                                             int G, int nj, int cap, float (&v)[NJ][8]) {
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    if (j >= nj) break;  // uniform over the item
    const int c = (c0 + G * j) * 8;
    float4 lo, hi;
    if (j == 0) {  // every lane: address clamped into the row, no branch
      const int ca = min(c, cap - 8);
      lo = *reinterpret_cast<const float4 *>(S + ro + ca);
      hi = *reinterpret_cast<const float4 *>(S + ro + ca + 4);
    } else if (c < m) {  // later chunks of long rows: only lanes inside the row
      lo = *reinterpret_cast<const float4 *>(S + ro + c);
      hi = *reinterpret_cast<const float4 *>(S + ro + c + 4);
    } else {
      lo = hi = make_float4(0.f, 0.f, 0.f, 0.f);
    }
    const float t[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) v[j][e] = c + e < m ? t[e] : -INFINITY;
  }
}

constexpr int kSmRing = 2;  // register sets of the softmax pipeline

template <int NJ, typename PT>
__global__ __launch_bounds__(256) void softmax_kernel(const float *__restrict__ S, PT *__restrict__ P,
                                                      const int32_t *__restrict__ off,
                                                      const int64_t *__restrict__ sbase,
                                                      const int32_t *__restrict__ items, int n_heads,
                                                      int causal) {
  const int seq = items[2 * blockIdx.x], row0 = items[2 * blockIdx.x + 1];
  const int n = off[seq + 1] - off[seq];
  const int64_t base = sbase[seq], block = score_block(n, causal != 0);
  const SoftmaxItem it = softmax_item(row0, n, n_heads, causal != 0);
  const int G = it.g;
  const int nj = (it.longest + 8 * G - 1) / (8 * G);  // chunks per lane its longest row needs
  // G = 128: a row on two wavefronts (uniform over the block)
  const bool pair = G > kWave;
  const int Gw = pair ? kWave : G;            // lanes of a row inside one wavefront
  const int rpw = kWave / Gw, rpp = 256 / G;  // rows per wavefront / per pass
  const int passes = (it.rows + rpp - 1) / rpp;
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x >> 6;
  const int sub = lane / Gw, c0 = (pair ? (wave & 1) * kWave : 0) + lane % Gw;
  const int wrow = pair ? wave >> 1 : wave * rpw + sub;  // the lane's row within a pass
  // pair exchange: [pass parity][max, sum][wavefront]
  __shared__ float xch[2][2][4];
  // row i of the item (clamped to its last row for the lanes past it): its
  // valid scores m (0 past the item), start ro and allocated length cap
  auto row_of = [&](int p, int &m, int64_t &ro, int &cap) {
    const int i = p * rpp + wrow, ic = min(i, it.rows - 1);
    int h, q;
    if (causal) {
      const int qn = it.qe - it.qs;
      h = it.h0 + ic / qn;
      q = it.qs + ic % qn;
    } else {
      h = (row0 + ic) / n;
      q = (row0 + ic) % n;
    }
    m = i < it.rows ? (causal ? q + 1 : n) : 0;
    ro = base + (int64_t)h * block + score_row_off(q, n, causal != 0);
    cap = causal ? score_ld(q + 1) : score_ld(n);
  };
  // a ring of kSmRing register sets: pass p computes in set p % kSmRing
  // while the loads of the next kSmRing - 1 passes are in flight
  float v[kSmRing][NJ][8];
  int m[kSmRing], cap[kSmRing];
  int64_t ro[kSmRing];
#pragma unroll
  for (int d = 0; d < kSmRing - 1; ++d) {
    if (d >= passes) break;
    row_of(d, m[d], ro[d], cap[d]);
    softmax_load<NJ>(S, ro[d], m[d], c0, G, nj, cap[d], v[d]);
  }
  for (int p0 = 0; p0 < passes; p0 += kSmRing) {
#pragma unroll
    for (int h = 0; h < kSmRing; ++h) {
      const int p = p0 + h;
      if (p >= passes) break;
      constexpr int kAhead = kSmRing - 1;
      const int nx = (h + kAhead) % kSmRing;
      if (p + kAhead < passes) {
        row_of(p + kAhead, m[nx], ro[nx], cap[nx]);
        softmax_load<NJ>(S, ro[nx], m[nx], c0, G, nj, cap[nx], v[nx]);
      }
      float mx = -INFINITY;
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        if (j >= nj) break;
#pragma unroll
        for (int e = 0; e < 8; ++e) mx = fmaxf(mx, v[h][j][e]);
      }
      mx = group_max(mx, Gw);
      if (pair) {  // block-uniform
        if (lane == 0) xch[p & 1][0][wave] = mx;
        __syncthreads();
        mx = fmaxf(mx, xch[p & 1][0][wave ^ 1]);
      }
      float sum = 0.f;
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        if (j >= nj) break;
        // exp(v - max) as 2^((v - max) log2 e): one v_exp_f32 each (masked
        // entries give exp2(-inf) = 0)
#pragma unroll
        for (int e = 0; e < 8; ++e) v[h][j][e] = __builtin_amdgcn_exp2f((v[h][j][e] - mx) * kLog2e);
        sum += ((v[h][j][0] + v[h][j][1]) + (v[h][j][2] + v[h][j][3])) +
               ((v[h][j][4] + v[h][j][5]) + (v[h][j][6] + v[h][j][7]));
      }
      sum = group_sum(sum, Gw);
      if (pair) {  // both wavefronts add the same two partial sums
        if (lane == 0) xch[p & 1][1][wave] = sum;
        __syncthreads();
        const float o = xch[p & 1][1][wave ^ 1];
        sum = (wave & 1) ? o + sum : sum + o;
      }
      const float inv = 1.0f / sum;  // one correctly rounded reciprocal per row
      PT *pr = P + ro[h];
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const int c = (c0 + G * j) * 8;
        if (j >= nj || c >= m[h]) continue;
        float o[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] = v[h][j][e] * inv;
        store8(pr + c, o);
      }
    }
  }
}

template <int NC, bool PRE_LN>
__global__ __launch_bounds__(256) void head_kernel(const float *__restrict__ x, int H,
                                                   const int32_t *__restrict__ off, int n_seqs,
                                                   const float *__restrict__ g,
                                                   const float *__restrict__ b, float eps,
                                                   const float *__restrict__ w,
                                                   const float *__restrict__ hb, float offset,
                                                   const int32_t *__restrict__ dest,
                                                   float *__restrict__ rewards) {
  const int lane = threadIdx.x & (kWave - 1);
  const int i = blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  if (i >= n_seqs) return;
  const int slot = dest ? dest[i] : i;
  if (slot < 0) return;  // a shared prompt: its continuations carry the rewards
  const int64_t t = off[i + 1] - 1;  // reward read at the end of the sequence
  const int c4n = H >> 2;
  float4 v[NC];
#pragma unroll
  for (int j = 0; j < NC; ++j) {
    const int c4 = lane + kWave * j;
    v[j] = c4 < c4n ? load4(x + t * H + 4 * c4) : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  if (PRE_LN) ln_row<NC>(v, lane, c4n, H, g, b, eps);
  float d = 0.f;
#pragma unroll
  for (int j = 0; j < NC; ++j) {
    const int c4 = lane + kWave * j;
    if (c4 < c4n) {
      const float4 ww = load4(w + 4 * c4);
      d += (v[j].x * ww.x + v[j].y * ww.y) + (v[j].z * ww.z + v[j].w * ww.w);
    }
  }
  d = wave_sum(d);
  if (lane == 0) rewards[slot] = (d + hb[0]) + offset;
}

// Best-of-N selection, one thread per prompt ("Learning to summarize from
// human feedback", Method adaptation: keep the candidate the reward model
// scores highest); a strict comparison keeps the lowest index among equals.
__global__ __launch_bounds__(256) void best_of_n_kernel(const float *__restrict__ rewards,
                                                        const int32_t *__restrict__ cstart,
                                                        int n_prompts, int32_t *__restrict__ best) {
  const int p = blockIdx.x * blockDim.x + threadIdx.x;
  if (p >= n_prompts) return;
  const int c0 = cstart[p], c1 = cstart[p + 1];
  int k = 0;
  float v = rewards[c0];
  for (int c = c0 + 1; c < c1; ++c) {
    const float r = rewards[c];
    if (r > v) {
      v = r;
      k = c - c0;
    }
  }
  best[p] = k;
}

// Smallest register-chunk count NC (float4 per lane) covering `cols`.
template <typename F>
hipError_t dispatch_nc(int cols, F &&f) {
  const int c4 = (cols + 3) / 4;
  if (c4 <= 64) return f(std::integral_constant<int, 1>{});
  if (c4 <= 128) return f(std::integral_constant<int, 2>{});
  if (c4 <= 256) return f(std::integral_constant<int, 4>{});
  if (c4 <= 512) return f(std::integral_constant<int, 8>{});
  if (c4 <= 1024) return f(std::integral_constant<int, 16>{});
  if (c4 <= 2048) return f(std::integral_constant<int, 32>{});
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_layernorm(bool act_bf16, const float *x, const float *sub, const float *g,
                            const float *b, int64_t rows, int cols, float eps, float *y, void *yb,
                            int ldb, int pad_cols, hipStream_t st) {
  if (rows <= 0) return hipSuccess;
  if (pad_cols < cols || pad_cols % 4 || (yb && pad_cols > ldb) ||
      pad_cols > 4 * kWave * ((cols / 4 + kWave - 1) / kWave))
    return hipErrorInvalidValue;
  const int padc4 = pad_cols / 4;
  // Four rows per wavefront for rows of 1025-2048 columns with nothing to
  // add, once there are enough rows for 16 such wavefronts per CU, one
  // otherwise.  Measured on one pass of each
  // largest stream: the decoder's pre-LN LayerNorm (2048 columns, affine
  // parameters twice the row's bytes) 282.5 -> 255.6-258.4 us; BERT-base's
  // residual-adding one (768 columns, parameters half the row's bytes) went
  // 160.6 -> 170.5 us with four rows (fewer wavefronts per SIMD), so it and
  // the narrower rows keep one row per wavefront.
  const bool many = rows >= (int64_t)4 * 256 * 16;  // 16 four-row wavefronts per CU
  auto go = [&](auto nc, auto rc) {
    constexpr int NC = decltype(nc)::value, R = decltype(rc)::value;
    const dim3 grid((unsigned)((rows + R * kRowsPerBlock - 1) / (R * kRowsPerBlock))), block(256);
    if (act_bf16) {
      auto k = sub ? layernorm_kernel<NC, uint16_t, true, R> : layernorm_kernel<NC, uint16_t, false, R>;
      k<<<grid, block, 0, st>>>(x, sub, g, b, rows, cols, eps, y, (uint16_t *)yb, ldb, padc4);
    } else {
      auto k = sub ? layernorm_kernel<NC, float, true, R> : layernorm_kernel<NC, float, false, R>;
      k<<<grid, block, 0, st>>>(x, sub, g, b, rows, cols, eps, y, (float *)yb, ldb, padc4);
    }
    return hipGetLastError();
  };
  return dispatch_nc(cols, [&](auto nc) {
    constexpr int NC = decltype(nc)::value;
    if (NC == 8 && many && sub == nullptr) return go(nc, std::integral_constant<int, 4>{});
    return go(nc, std::integral_constant<int, 1>{});
  });
}

hipError_t launch_zero_cols(void *base, int64_t ld_bytes, int rows, int64_t c0_bytes,
                            int64_t c1_bytes, hipStream_t st) {
  if (rows <= 0 || c1_bytes <= c0_bytes) return hipSuccess;
  if (c0_bytes % 4 || c1_bytes % 4 || ld_bytes % 4 || c1_bytes > ld_bytes) return hipErrorInvalidValue;
  const int words = (int)((c1_bytes - c0_bytes) / 4);
  const dim3 grid((unsigned)((rows + kRowsPerBlock - 1) / kRowsPerBlock)), block(256);
  zero_cols_kernel<<<grid, block, 0, st>>>(static_cast<char *>(base) + c0_bytes, ld_bytes / 4, rows, words);
  return hipGetLastError();
}

hipError_t launch_embed(bool w_bf16, bool act_bf16, bool ln, const int32_t *ids, const Ragged &r,
                        const void *tok, const void *pos, int vocab, int H, const float *g,
                        const float *b, float eps, float *x, void *xb, int ldb, int *flag,
                        hipStream_t st) {
  if (r.n_tokens <= 0) return hipSuccess;
  const dim3 grid((r.n_tokens + kRowsPerBlock - 1) / kRowsPerBlock), block(256);
  return dispatch_nc(H, [&](auto nc) {
    constexpr int NC = decltype(nc)::value;
    if (w_bf16 != act_bf16) return hipErrorInvalidValue;
    if (w_bf16) {
      auto k = ln ? embed_kernel<NC, uint16_t, true, uint16_t> : embed_kernel<NC, uint16_t, false, uint16_t>;
      k<<<grid, block, 0, st>>>(ids, r.off, r.src, r.plen, r.n_seqs, r.n_tokens, (const uint16_t *)tok,
                                (const uint16_t *)pos, vocab, H, g, b, eps, x, (uint16_t *)xb, ldb,
                                ldb / 4, flag);
    } else {
      auto k = ln ? embed_kernel<NC, float, true, float> : embed_kernel<NC, float, false, float>;
      k<<<grid, block, 0, st>>>(ids, r.off, r.src, r.plen, r.n_seqs, r.n_tokens, (const float *)tok,
                                (const float *)pos, vocab, H, g, b, eps, x, (float *)xb, ldb,
                                ldb / 4, flag);
    }
    return hipGetLastError();
  });
}

hipError_t launch_softmax(bool p_bf16, const float *S, void *P, const Ragged &r, int n_heads,
                          bool causal, hipStream_t st) {
  if (r.n_sm_items <= 0) return hipSuccess;
  const dim3 block(256);
  // items [0, n_sm_narrow): one chunk per lane (rows of at most 512 scores,
  // causal rows of at most 1024 on two wavefronts); the rest: 64 lanes per
  // row and as many chunks as the longest row needs
  auto go = [&](auto njc, int first, int count) {
    constexpr int NJ = decltype(njc)::value;
    if (count <= 0) return hipSuccess;
    const int32_t *it = r.sm_items + 2 * first;
    if (p_bf16)
      softmax_kernel<NJ, uint16_t><<<count, block, 0, st>>>(S, (uint16_t *)P, r.off, r.sbase, it,
                                                             n_heads, causal ? 1 : 0);
    else
      softmax_kernel<NJ, float><<<count, block, 0, st>>>(S, (float *)P, r.off, r.sbase, it, n_heads,
                                                          causal ? 1 : 0);
    return hipGetLastError();
  };
  hipError_t e = go(std::integral_constant<int, 1>{}, 0, r.n_sm_narrow);
  if (e != hipSuccess) return e;
  const int first = r.n_sm_narrow, count = r.n_sm_items - r.n_sm_narrow;
  const int nc = (r.max_len + 7) / 8;  // eight-score chunks of the longest row
  const int nj = (nc + 63) / 64;       // chunks per lane of 64-lane rows
  if (count <= 0) return hipSuccess;
  if (nj <= 2) return go(std::integral_constant<int, 2>{}, first, count);
  if (nj <= 3) return go(std::integral_constant<int, 3>{}, first, count);
  if (nj <= 4) return go(std::integral_constant<int, 4>{}, first, count);
  if (nj <= 8) return go(std::integral_constant<int, 8>{}, first, count);
  return hipErrorInvalidValue;
}

hipError_t launch_head(bool pre_ln, const float *x, int H, const Ragged &r, const float *g,
                       const float *b, float eps, const float *w, const float *hb, float offset,
                       float *rewards, hipStream_t st) {
  if (r.n_seqs <= 0) return hipSuccess;
  const dim3 grid((r.n_seqs + kRowsPerBlock - 1) / kRowsPerBlock), block(256);
  return dispatch_nc(H, [&](auto nc) {
    constexpr int NC = decltype(nc)::value;
    if (pre_ln)
      head_kernel<NC, true><<<grid, block, 0, st>>>(x, H, r.off, r.n_seqs, g, b, eps, w, hb, offset,
                                                    r.dest, rewards);
    else
      head_kernel<NC, false><<<grid, block, 0, st>>>(x, H, r.off, r.n_seqs, g, b, eps, w, hb,
                                                     offset, r.dest, rewards);
    return hipGetLastError();
  });
}

hipError_t launch_best_of_n(const float *rewards, const int32_t *cstart, int n_prompts,
                            int32_t *best, hipStream_t st) {
  if (n_prompts <= 0) return hipSuccess;
  best_of_n_kernel<<<(n_prompts + 255) / 256, 256, 0, st>>>(rewards, cstart, n_prompts, best);
  return hipGetLastError();
}

namespace {
// One block per gathered row: 4-byte words of the two row pieces.
__global__ __launch_bounds__(256) void gather_rows_kernel(const uint32_t *__restrict__ a, int ap, uint32_t *__restrict__ ad,
                                                          int adp, int aw, const uint32_t *__restrict__ c, int cp,
                                                          uint32_t *__restrict__ cd, int cdp, int cw,
                                                          const int32_t *__restrict__ rows) {
  const int i = blockIdx.x;
  const int64_t r = rows[i];
  for (int k = threadIdx.x; k < aw; k += blockDim.x) ad[(int64_t)i * adp + k] = a[r * ap + k];
  for (int k = threadIdx.x; k < cw; k += blockDim.x) cd[(int64_t)i * cdp + k] = c[r * cp + k];
}
}  // namespace

namespace {
// LayerNorm of fp32 rows into the split-operand layout (split_off): one block
// per row, mean and variance over the row in two passes, fixed reduction
// order.  For the refinement rows, which feed the split GEMMs.
__global__ __launch_bounds__(256) void layernorm_split_kernel(const float *__restrict__ x,
                                                              const float *__restrict__ g,
                                                              const float *__restrict__ b, int cols,
                                                              float eps, uint16_t *__restrict__ out) {
  __shared__ float red[2][4];
  const int64_t row = blockIdx.x;
  const int t = threadIdx.x, lane = t % kWave, wv = t / kWave, c4 = cols / 4;
  const float4 *xr = reinterpret_cast<const float4 *>(x + row * cols);
  float s = 0.f;
  for (int c = t; c < c4; c += 256) {
    const float4 v = xr[c];
    s += (v.x + v.y) + (v.z + v.w);
  }
  s = wave_sum(s);
  if (lane == 0) red[0][wv] = s;
  __syncthreads();
  const float mean = ((red[0][0] + red[0][1]) + (red[0][2] + red[0][3])) / cols;
  float q = 0.f;
  for (int c = t; c < c4; c += 256) {
    const float4 v = xr[c];
    const float d0 = v.x - mean, d1 = v.y - mean, d2 = v.z - mean, d3 = v.w - mean;
    q += (d0 * d0 + d1 * d1) + (d2 * d2 + d3 * d3);
  }
  q = wave_sum(q);
  if (lane == 0) red[1][wv] = q;
  __syncthreads();
  const float rstd = rsqrtf(((red[1][0] + red[1][1]) + (red[1][2] + red[1][3])) / cols + eps);
  for (int c = t; c < c4; c += 256) {
    const float4 v = xr[c], gg = reinterpret_cast<const float4 *>(g)[c],
                 bb = reinterpret_cast<const float4 *>(b)[c];
    const float y[4] = {(v.x - mean) * rstd * gg.x + bb.x, (v.y - mean) * rstd * gg.y + bb.y,
                        (v.z - mean) * rstd * gg.z + bb.z, (v.w - mean) * rstd * gg.w + bb.w};
    uint2 hi, lo;
    split4(y, hi, lo);
    *reinterpret_cast<uint2 *>(out + split_off(row, 4 * c, cols, 0)) = hi;
    *reinterpret_cast<uint2 *>(out + split_off(row, 4 * c, cols, 1)) = lo;
  }
}
// fp32 rows into the split-operand layout, 4 elements per thread; rows in
// [M, 32 ceil(M / 32)) become zeros.
__global__ __launch_bounds__(256) void split_rows_kernel(const float *__restrict__ a, int lda, int M,
                                                         int K, int64_t n4, uint16_t *__restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n4) return;
  const int k4 = K / 4;
  const int64_t m = i / k4;
  const int c = (int)(i % k4);
  float v[4] = {0.f, 0.f, 0.f, 0.f};
  if (m < M) {
    const float4 x = *reinterpret_cast<const float4 *>(a + m * lda + 4 * c);
    v[0] = x.x, v[1] = x.y, v[2] = x.z, v[3] = x.w;
  }
  uint2 hi, lo;
  split4(v, hi, lo);
  *reinterpret_cast<uint2 *>(out + split_off(m, 4 * c, K, 0)) = hi;
  *reinterpret_cast<uint2 *>(out + split_off(m, 4 * c, K, 1)) = lo;
}
}  // namespace

hipError_t launch_split_rows(const float *a, int lda, int M, int K, uint16_t *out, hipStream_t st) {
  if (M <= 0) return hipSuccess;
  if (K <= 0 || K % 16 || lda < K || lda % 4) return hipErrorInvalidValue;
  const int64_t n4 = (int64_t)(M + 31) / 32 * 32 * (K / 4);
  split_rows_kernel<<<(unsigned)((n4 + 255) / 256), 256, 0, st>>>(a, lda, M, K, n4, out);
  return hipGetLastError();
}

hipError_t launch_layernorm_split(const float *x, const float *g, const float *b, int rows, int cols,
                                  float eps, uint16_t *out, hipStream_t st) {
  if (rows <= 0) return hipSuccess;
  if (cols <= 0 || cols % 16) return hipErrorInvalidValue;
  layernorm_split_kernel<<<rows, 256, 0, st>>>(x, g, b, cols, eps, out);
  return hipGetLastError();
}

hipError_t launch_gather_rows(const void *a_src, int a_pitch, void *a_dst, int a_dpitch, int a_bytes,
                              const void *c_src, int c_pitch, void *c_dst, int c_dpitch, int c_bytes,
                              const int32_t *rows, int n, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  if ((a_pitch | a_dpitch | a_bytes | c_pitch | c_dpitch | c_bytes) & 3) return hipErrorInvalidValue;
  gather_rows_kernel<<<n, 256, 0, st>>>((const uint32_t *)a_src, a_pitch / 4, (uint32_t *)a_dst, a_dpitch / 4,
                                        a_bytes / 4, (const uint32_t *)c_src, c_pitch / 4, (uint32_t *)c_dst,
                                        c_dpitch / 4, c_bytes / 4, rows);
  return hipGetLastError();
}

}  // namespace es
