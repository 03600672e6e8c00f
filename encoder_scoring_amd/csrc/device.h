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
//   erfc(x) = t exp(-x^2 + P(t)),  t = 1 / (1 + x/2),  x >= 0,
// and 1 + erf(x) = 2 - erfc(x) for x >= 0, erfc(-x) for x < 0, so the
// negative tail keeps its relative accuracy (no cancellation).  Measured in
// float32 over z in [-12, 12]: relative error below 3e-6 wherever
// |GELU(z)| > 1e-6, i.e. far below one bf16 step (2^-8).
__device__ __forceinline__ float gelu_erf_bf16out(float z) {
  const float x = fabsf(z) * 0.70710678118654752440f;
  const float t = __builtin_amdgcn_rcpf(1.0f + 0.5f * x);
  float p = 0.17087277f;
  p = fmaf(p, t, -0.82215223f);
  p = fmaf(p, t, 1.48851587f);
  p = fmaf(p, t, -1.13520398f);
  p = fmaf(p, t, 0.27886807f);
  p = fmaf(p, t, -0.18628806f);
  p = fmaf(p, t, 0.09678418f);
  p = fmaf(p, t, 0.37409196f);
  p = fmaf(p, t, 1.00002368f);
  p = fmaf(p, t, -1.26551223f);
  const float q = t * __builtin_amdgcn_exp2f((p - x * x) * 1.44269504088896340736f);  // erfc(|x|)
  return 0.5f * z * (z >= 0.0f ? 2.0f - q : q);
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
