// Masked attention over the packed, ragged batch, in two kernels around the
// Softmax row reduction (TurboTransformers review, Proposed method: Softmax
// is its own per-row "batch reduction" kernel):
//   scores:  S_ih[q, k] = (q_q . k_k) / sqrt(d)  for keys k of the same
//            sequence (all k < n_i, or k <= q when causal), fp32;
//   P = softmax(S) row by row (rowops.hip);
//   context: ctx[q, h*dp + e] = sum_k P_ih[q, k] v_k[h*dp + e].
// Work is a list of (sequence, 32-query-row tile) items built on the host,
// longest sequences first, times the heads on the second grid axis, so no
// block is spent on padding.  Score blocks of sequence i are n_i x ld_i
// (ld_i = n_i rounded up to 8) per head, packed back to back.
#include "device.h"
#include "kernels.h"

namespace es {

namespace {

template <typename Act, int DP>
__global__ __launch_bounds__(256) void scores_kernel(const Act *__restrict__ qkv, int ldq,
                                                     int n_heads, float scale, int causal,
                                                     const int32_t *__restrict__ off,
                                                     const int64_t *__restrict__ sbase,
                                                     const int32_t *__restrict__ items,
                                                     float *__restrict__ S) {
  __shared__ float sQ[kQTile][DP + 1];
  __shared__ float sK[64][DP + 1];
  const int item = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
  const int seq = items[2 * item], q0 = items[2 * item + 1];
  const int64_t t0 = off[seq];
  const int n = off[seq + 1] - (int)t0;
  const int ld = score_ld(n);
  const int64_t base = sbase[seq] + (int64_t)h * n * ld;
  const Act *Q = qkv + t0 * ldq + h * DP;
  const Act *Kp = qkv + t0 * ldq + (n_heads + h) * DP;
  for (int e = tid; e < kQTile * DP; e += 256) {
    const int r = e / DP, c = e % DP, q = q0 + r;
    sQ[r][c] = q < n ? to_f(Q[(int64_t)q * ldq + c]) : 0.f;
  }
  const int kend = causal ? min(n, q0 + kQTile) : n;
  const int kc = tid & 63, rg = (tid >> 6) * 8;
  for (int k0 = 0; k0 < kend; k0 += 64) {
    __syncthreads();
    for (int e = tid; e < 64 * DP; e += 256) {
      const int r = e / DP, c = e % DP, k = k0 + r;
      sK[r][c] = k < n ? to_f(Kp[(int64_t)k * ldq + c]) : 0.f;
    }
    __syncthreads();
    float acc[8] = {};
#pragma unroll 8
    for (int c = 0; c < DP; ++c) {
      const float kv = sK[kc][c];
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] = fmaf(sQ[rg + i][c], kv, acc[i]);
    }
    const int k = k0 + kc;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int q = q0 + rg + i;
      if (q < n && k < n && (!causal || k <= q)) S[base + (int64_t)q * ld + k] = acc[i] * scale;
    }
  }
}

template <typename Act, typename PT, int DP>
__global__ __launch_bounds__(256) void pv_kernel(const PT *__restrict__ P, const Act *__restrict__ qkv,
                                                 int ldq, int n_heads, int causal,
                                                 const int32_t *__restrict__ off,
                                                 const int64_t *__restrict__ sbase,
                                                 const int32_t *__restrict__ items,
                                                 Act *__restrict__ ctx, int ldc) {
  constexpr int RS = 256 / DP, NR = kQTile / RS;
  __shared__ float sP[kQTile][64 + 1];
  __shared__ float sV[64][DP + 1];
  const int item = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
  const int seq = items[2 * item], q0 = items[2 * item + 1];
  const int64_t t0 = off[seq];
  const int n = off[seq + 1] - (int)t0;
  const int ld = score_ld(n);
  const int64_t base = sbase[seq] + (int64_t)h * n * ld;
  const Act *V = qkv + t0 * ldq + (2 * n_heads + h) * DP;
  const int e = tid % DP, r0 = tid / DP;
  float acc[NR] = {};
  const int kend = causal ? min(n, q0 + kQTile) : n;
  for (int k0 = 0; k0 < kend; k0 += 64) {
    __syncthreads();
    for (int x = tid; x < kQTile * 64; x += 256) {
      const int r = x >> 6, c = x & 63, q = q0 + r, k = k0 + c;
      const bool ok = q < n && k < n && (!causal || k <= q);
      sP[r][c] = ok ? to_f(P[base + (int64_t)q * ld + k]) : 0.f;
    }
    for (int x = tid; x < 64 * DP; x += 256) {
      const int r = x / DP, c = x % DP, k = k0 + r;
      sV[r][c] = k < n ? to_f(V[(int64_t)k * ldq + c]) : 0.f;
    }
    __syncthreads();
#pragma unroll 4
    for (int kk = 0; kk < 64; ++kk) {
      const float v = sV[kk][e];
#pragma unroll
      for (int j = 0; j < NR; ++j) acc[j] = fmaf(sP[r0 + j * RS][kk], v, acc[j]);
    }
  }
#pragma unroll
  for (int j = 0; j < NR; ++j) {
    const int q = q0 + r0 + j * RS;
    if (q < n) ctx[(t0 + q) * ldc + h * DP + e] = from_f<Act>(acc[j]);
  }
}

template <typename F>
hipError_t dispatch_dp(int dp, F &&f) {
  switch (dp) {
    case 16: return f(std::integral_constant<int, 16>{});
    case 32: return f(std::integral_constant<int, 32>{});
    case 64: return f(std::integral_constant<int, 64>{});
    case 128: return f(std::integral_constant<int, 128>{});
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_scores(bool act_bf16, const void *qkv, int ldq, int n_heads, int dp, float scale,
                         bool causal, const Ragged &r, float *S, hipStream_t st) {
  if (r.n_items <= 0) return hipSuccess;
  const dim3 grid(r.n_items, n_heads), block(256);
  return dispatch_dp(dp, [&](auto dpc) {
    constexpr int DP = decltype(dpc)::value;
    if (act_bf16)
      scores_kernel<uint16_t, DP><<<grid, block, 0, st>>>((const uint16_t *)qkv, ldq, n_heads, scale,
                                                          causal ? 1 : 0, r.off, r.sbase, r.items, S);
    else
      scores_kernel<float, DP><<<grid, block, 0, st>>>((const float *)qkv, ldq, n_heads, scale,
                                                       causal ? 1 : 0, r.off, r.sbase, r.items, S);
    return hipGetLastError();
  });
}

hipError_t launch_pv(bool act_bf16, const void *P, const void *qkv, int ldq, int n_heads, int dp,
                     bool causal, const Ragged &r, void *ctx, int ldc, hipStream_t st) {
  if (r.n_items <= 0) return hipSuccess;
  const dim3 grid(r.n_items, n_heads), block(256);
  return dispatch_dp(dp, [&](auto dpc) {
    constexpr int DP = decltype(dpc)::value;
    if (act_bf16)
      pv_kernel<uint16_t, uint16_t, DP><<<grid, block, 0, st>>>(
          (const uint16_t *)P, (const uint16_t *)qkv, ldq, n_heads, causal ? 1 : 0, r.off, r.sbase,
          r.items, (uint16_t *)ctx, ldc);
    else
      pv_kernel<float, float, DP><<<grid, block, 0, st>>>((const float *)P, (const float *)qkv, ldq,
                                                          n_heads, causal ? 1 : 0, r.off, r.sbase,
                                                          r.items, (float *)ctx, ldc);
    return hipGetLastError();
  });
}

}  // namespace es
