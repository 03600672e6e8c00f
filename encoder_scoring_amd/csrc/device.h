// Device-side helpers shared by the gfx950 kernels of libencscore.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace es {

constexpr int kWave = 64;  // CDNA wavefront width

// bf16 is stored as raw 16-bit patterns; conversion rounds to nearest even.
__device__ __forceinline__ float bf2f(uint16_t b) { return __uint_as_float(((uint32_t)b) << 16); }

// float -> bf16 bits, round to nearest even (gfx950's v_cvt_pk_bf16_f32; a
// NaN stays a quiet NaN).
__device__ __forceinline__ uint16_t f2bf(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }

// Two floats -> packed bf16 bits (lo in bits 0..15), one conversion instruction.
__device__ __forceinline__ uint32_t f2bf2(float lo, float hi) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// Block ids are dealt round-robin to the 8 XCDs (each with its own L2):
// the block of id bid on a grid of nblk takes logical index
// xcd_contiguous(bid, nblk), so each XCD runs one contiguous run of logical
// indices and neighbouring work items share that XCD's L2.
__device__ __forceinline__ int xcd_contiguous(int bid, int nblk) {
  const int per = (nblk + 7) / 8, xcd = bid & 7, loc = bid >> 3;
  const int full = nblk - (per - 1) * 8;  // XCDs that receive `per` blocks
  return xcd < full ? xcd * per + loc : full * per + (xcd - full) * (per - 1) + loc;
}

// Split-operand layout of an fp32 matrix [rows, K] (K a multiple of 16) for
// the refinement GEMMs: each element a as the bf16 pair hi = bf16(a), lo =
// bf16(a - hi), stored in the order the 32 x 32 x 16 MFMA takes its operand.
// For row tile t (rows 32 t ..), k-step s (columns 16 s ..) and half h (0 hi,
// 1 lo) a block of 64 lanes x 8 bf16; lane 32 f + r holds row 32 t + r,
// columns 16 s + 8 f .. + 8.  So one wavefront load of 16 bytes per lane
// reads 1 KB of contiguous memory.  Offset (bf16 units) of element (m, k):
__device__ __forceinline__ int64_t split_off(int64_t m, int k, int K, int h) {
  return ((((m >> 5) * (K >> 4) + (k >> 4)) * 2 + h) * 64 + ((k >> 3) & 1) * 32 + (m & 31)) * 8 + (k & 7);
}

// hi / lo bf16 bits of 4 consecutive floats (8 bytes each).
__device__ __forceinline__ void split4(const float (&v)[4], uint2 &hi, uint2 &lo) {
  float r[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) r[e] = v[e] - bf2f(f2bf(v[e]));
  hi = make_uint2(f2bf2(v[0], v[1]), f2bf2(v[2], v[3]));
  lo = make_uint2(f2bf2(r[0], r[1]), f2bf2(r[2], r[3]));
}

__device__ __forceinline__ float to_f(float v) { return v; }
__device__ __forceinline__ float to_f(uint16_t v) { return bf2f(v); }

template <typename T>
__device__ __forceinline__ T from_f(float v);
template <>
__device__ __forceinline__ float from_f<float>(float v) { return v; }
template <>
__device__ __forceinline__ uint16_t from_f<uint16_t>(float v) { return f2bf(v); }

// Butterfly reductions: every lane ends with the bitwise-identical result and
// the order of additions is fixed, so results are reproducible run to run.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

// Reductions inside aligned groups of g lanes (g a power of two <= 64).
__device__ __forceinline__ float group_sum(float v, int g) {
  for (int o = g >> 1; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

__device__ __forceinline__ float group_max(float v, int g) {
  for (int o = g >> 1; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

// GELU in its exact form z * Phi(z) = z/2 * (1 + erf(z / sqrt(2))).
__device__ __forceinline__ float gelu_erf(float z) {
  return 0.5f * z * (1.0f + erff(z * 0.70710678118654752440f));
}

// The same GELU for outputs stored as bf16, with erfc from the Chebyshev fit
// of Numerical Recipes (Press et al., 2nd ed., section 6.2, "erfcc":
// fractional error below 1.2e-7 for every argument):
//   erfc(x) = t exp(-x^2 + P(t)),  t = 1 / (1 + x/2),  x = |z| / sqrt(2),
// evaluated in base 2 with the constants folded in: with y = x sqrt(log2 e),
//   z erfc(x) / 2 = z t 2^(-y^2 + P'(t)),  P' = log2(e) P - 1,
// and GELU(z) = max(z, 0) - |z erfc(x) / 2|: z - h for z >= 0 (h >= 0),
// h for z < 0 (h <= 0) -- so the negative tail keeps its relative accuracy
// (no cancellation).  One reciprocal, one exp2, 9 + 6 fma / mul / max.
// Measured in float32 over z in [-12, 12]: relative error below 3.4e-6
// wherever |GELU(z)| > 1e-6, far below one bf16 step (2^-8).  Non-finite
// z gives NaN.
__device__ __forceinline__ float gelu_erf_bf16out(float z) {
  const float y = fabsf(z) * 8.493217826e-01f;  // |z| / sqrt(2) * sqrt(log2 e)
  const float t = __builtin_amdgcn_rcpf(fmaf(y, 4.162773192e-01f, 1.0f));  // 1 / (1 + x / 2)
  float p = 2.465173006e-01f;  // the erfcc coefficients times log2 e
  p = fmaf(p, t, -1.186114907e+00f);
  p = fmaf(p, t, 2.147474527e+00f);
  p = fmaf(p, t, -1.637753129e+00f);
  p = fmaf(p, t, 4.023215771e-01f);
  p = fmaf(p, t, -2.687568665e-01f);
  p = fmaf(p, t, 1.396300495e-01f);
  p = fmaf(p, t, 5.397006273e-01f);
  p = fmaf(p, t, 1.442729235e+00f);
  p = fmaf(p, t, -2.825748205e+00f);  // log2(e) (-1.26551223) - 1: the factor 1/2
  const float h = z * (t * __builtin_amdgcn_exp2f(fmaf(-y, y, p)));  // z erfc(x) / 2
  return fmaxf(z, 0.0f) - fabsf(h);
}

// Sequence that owns packed token t: the last i with off[i] <= t.
__device__ __forceinline__ int seq_of_token(const int32_t *off, int n_seqs, int t) {
  int lo = 0, hi = n_seqs - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (off[mid] <= t) lo = mid; else hi = mid - 1;
  }
  return lo;
}

}  // namespace es
