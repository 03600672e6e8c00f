// Row kernels: embedding (+LN), LayerNorm, ragged Softmax, reward head.
//
// TurboTransformers review (Proposed method): Softmax and LayerNorm are the
// hot spots besides the GEMMs and are computed as parallel per-row ("batch")
// reductions.  On gfx950 each row (or group of short rows) is owned by one
// 64-lane wavefront: coalesced 16-byte loads straight into registers, one
// pass over HBM in and out, reductions by butterfly shuffles inside the
// wavefront, no barriers.
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
// it writes any of it.
template <int NC, typename OutB, bool ADD>
__global__ __launch_bounds__(256) void layernorm_kernel(const float *x, const float *sub,
                                                        const float *__restrict__ g,
                                                        const float *__restrict__ b, int64_t rows,
                                                        int cols, float eps, float *y, OutB *yb,
                                                        int ldb, int padc4) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int c4n = cols >> 2;
  const float *xr = x + row * cols;
  // every load is issued before any is used, at an in-bounds chunk (lanes
  // past the row end re-read its last chunk and are zeroed below): loads
  // under a per-chunk branch made the compiler wait for each chunk's pair
  // before issuing the next, one memory round trip per chunk
  float4 v[NC], u[NC], gg[NC], bb[NC];
#pragma unroll
  for (int j = 0; j < NC; ++j) {
    const int c4 = min(lane + kWave * j, c4n - 1);
    v[j] = load4(xr + 4 * c4);
    if (ADD) u[j] = load4(sub + row * cols + 4 * c4);
  }
  ln_load_affine<NC>(gg, bb, lane, c4n, g, b);
#pragma unroll
  for (int j = 0; j < NC; ++j) {  // selects, no branches
    const bool in = lane + kWave * j < c4n;
    if (ADD) {
      v[j].x += u[j].x; v[j].y += u[j].y; v[j].z += u[j].z; v[j].w += u[j].w;
    }
    v[j].x = in ? v[j].x : 0.f;
    v[j].y = in ? v[j].y : 0.f;
    v[j].z = in ? v[j].z : 0.f;
    v[j].w = in ? v[j].w : 0.f;
  }
  ln_apply<NC>(v, gg, bb, lane, c4n, cols, eps);
#pragma unroll
  for (int j = 0; j < NC; ++j) {
    const int c4 = lane + kWave * j;
    if (c4 < c4n) {
      if (y) store4(y + row * cols + 4 * c4, v[j]);
      if (yb) store4(yb + row * ldb + 4 * c4, v[j]);
    } else if (yb && c4 < padc4) {  // zero padding columns of the GEMM input
      store4(yb + row * ldb + 4 * c4, make_float4(0.f, 0.f, 0.f, 0.f));
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

// Softmax over the ragged score rows.  One item covers a run of rows of one
// sequence's [A * n, ld] score block (all heads; rows of equal length n, or
// q + 1 when causal).  Each row is owned by G lanes (G from its length) that
// read it as float4 chunks straight into registers; both passes of rows are
// loaded before any reduction so two rows per lane group are in flight.
// Max and sum reduce by butterfly shuffles within the G-lane group.
template <int NJ, typename PT>
__global__ __launch_bounds__(256) void softmax_kernel(const float *__restrict__ S, PT *__restrict__ P,
                                                      const int32_t *__restrict__ off,
                                                      const int64_t *__restrict__ sbase,
                                                      const int32_t *__restrict__ items, int n_heads,
                                                      int causal) {
  const int seq = items[2 * blockIdx.x], row0 = items[2 * blockIdx.x + 1];
  const int n = off[seq + 1] - off[seq];
  const int ld = score_ld(n);
  const int64_t base = sbase[seq];
  const int G = softmax_lanes(n), rpw = kWave / G;
  const int row_end = min(row0 + softmax_rows_per_item(n), n_heads * n);
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x >> 6;
  const int sub = lane / G, c0 = lane % G;
  float4 v[kSoftmaxPasses][NJ];
  int m[kSoftmaxPasses];
  int64_t ro[kSoftmaxPasses];
#pragma unroll
  for (int p = 0; p < kSoftmaxPasses; ++p) {
    const int r = row0 + (p * 4 + wave) * rpw + sub;
    m[p] = r < row_end ? (causal ? r % n + 1 : n) : 0;  // valid scores of row r
    ro[p] = base + (int64_t)r * ld;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int c = (c0 + G * j) * 4;
      v[p][j] = c < m[p] ? *reinterpret_cast<const float4 *>(S + ro[p] + c)
                         : make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
    }
  }
#pragma unroll
  for (int p = 0; p < kSoftmaxPasses; ++p) {
    float mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int c = (c0 + G * j) * 4;
      if (c < m[p]) mx = fmaxf(mx, v[p][j].x);
      if (c + 1 < m[p]) mx = fmaxf(mx, v[p][j].y);
      if (c + 2 < m[p]) mx = fmaxf(mx, v[p][j].z);
      if (c + 3 < m[p]) mx = fmaxf(mx, v[p][j].w);
    }
    mx = group_max(mx, G);
    float sum = 0.f;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int c = (c0 + G * j) * 4;
      // exp(v - max) as 2^((v - max) log2 e): one v_exp_f32 each
      v[p][j].x = c < m[p] ? __builtin_amdgcn_exp2f((v[p][j].x - mx) * kLog2e) : 0.f;
      v[p][j].y = c + 1 < m[p] ? __builtin_amdgcn_exp2f((v[p][j].y - mx) * kLog2e) : 0.f;
      v[p][j].z = c + 2 < m[p] ? __builtin_amdgcn_exp2f((v[p][j].z - mx) * kLog2e) : 0.f;
      v[p][j].w = c + 3 < m[p] ? __builtin_amdgcn_exp2f((v[p][j].w - mx) * kLog2e) : 0.f;
      sum += (v[p][j].x + v[p][j].y) + (v[p][j].z + v[p][j].w);
    }
    sum = group_sum(sum, G);
    PT *pr = P + ro[p];
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int c = (c0 + G * j) * 4;
      if (c >= m[p]) continue;
      const float4 o = make_float4(v[p][j].x / sum, v[p][j].y / sum, v[p][j].z / sum, v[p][j].w / sum);
      if (c + 3 < m[p]) {
        store4(pr + c, o);
      } else {
        pr[c] = from_f<PT>(o.x);
        if (c + 1 < m[p]) pr[c + 1] = from_f<PT>(o.y);
        if (c + 2 < m[p]) pr[c + 2] = from_f<PT>(o.z);
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
  const dim3 grid((unsigned)((rows + kRowsPerBlock - 1) / kRowsPerBlock)), block(256);
  return dispatch_nc(cols, [&](auto nc) {
    constexpr int NC = decltype(nc)::value;
    if (act_bf16) {
      auto k = sub ? layernorm_kernel<NC, uint16_t, true> : layernorm_kernel<NC, uint16_t, false>;
      k<<<grid, block, 0, st>>>(x, sub, g, b, rows, cols, eps, y, (uint16_t *)yb, ldb, padc4);
    } else {
      auto k = sub ? layernorm_kernel<NC, float, true> : layernorm_kernel<NC, float, false>;
      k<<<grid, block, 0, st>>>(x, sub, g, b, rows, cols, eps, y, (float *)yb, ldb, padc4);
    }
    return hipGetLastError();
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
  const dim3 grid(r.n_sm_items), block(256);
  const int nc = (r.max_len + 3) / 4;
  const int nj = nc <= 64 ? 1 : (nc + 63) / 64;
  auto go = [&](auto njc) {
    constexpr int NJ = decltype(njc)::value;
    if (p_bf16)
      softmax_kernel<NJ, uint16_t><<<grid, block, 0, st>>>(S, (uint16_t *)P, r.off, r.sbase,
                                                            r.sm_items, n_heads, causal ? 1 : 0);
    else
      softmax_kernel<NJ, float><<<grid, block, 0, st>>>(S, (float *)P, r.off, r.sbase, r.sm_items,
                                                         n_heads, causal ? 1 : 0);
    return hipGetLastError();
  };
  if (nj <= 1) return go(std::integral_constant<int, 1>{});
  if (nj <= 2) return go(std::integral_constant<int, 2>{});
  if (nj <= 4) return go(std::integral_constant<int, 4>{});
  if (nj <= 8) return go(std::integral_constant<int, 8>{});
  if (nj <= 16) return go(std::integral_constant<int, 16>{});
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
