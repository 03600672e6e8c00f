// Dense GEMMs of the hot path: QKV, attention output, FFN1, FFN2.
//
//   out[m, n] = epilogue( sum_k A[m, k] * W[n, k] + bias[n] )
//
// A is the packed activation matrix [tokens, K] (no padding between
// sequences), W a weight matrix stored [out, in]; both are K-contiguous, which
// is exactly the operand layout of the CDNA matrix cores.  TurboTransformers
// review (Abstract): the BLAS GEMMs are the main hot spot, and tensor-core
// mixed precision is used "without accuracy loss" -- here bf16 operands with
// fp32 accumulation on gfx950 MFMA (v_mfma_f32_32x32x16_bf16).
//
// Epilogues fuse what follows each GEMM: bias (QKV), bias + exact GELU (FFN1),
// bias + fp32 residual (attention output, FFN2).
#include "device.h"
#include "kernels.h"

namespace es {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

template <int EPI>
__device__ __forceinline__ void epi_store(void *out, const float *__restrict__ res, int ldc,
                                          int64_t m, int n, float v) {
  if (EPI == kEpiBias) {
    static_cast<uint16_t *>(out)[m * ldc + n] = f2bf(v);
  } else if (EPI == kEpiGelu) {
    static_cast<uint16_t *>(out)[m * ldc + n] = f2bf(gelu_erf(v));
  } else if (EPI == kEpiResidual) {
    static_cast<float *>(out)[m * ldc + n] = v + res[m * ldc + n];
  } else {
    static_cast<float *>(out)[m * ldc + n] = v;
  }
}

// ---------------------------------------------------------------- bf16 MFMA
//
// Block tile BM x BN, K step 64, 4 wavefronts in a 2 x 2 grid, each owning a
// (BM/2) x (BN/2) sub-tile of 32 x 32 MFMA tiles.  Tiles of A and W are
// staged through LDS, double-buffered: the global loads of step k+1 are in
// flight while the matrix cores work on step k, and one barrier per step
// separates the buffers.  LDS rows are padded to 72 bf16 (144 B) so the
// 16-byte fragment reads of a wavefront hit distinct banks.
template <int BM, int BN, int EPI>
__global__ __launch_bounds__(256) void gemm_bf16_kernel(const uint16_t *__restrict__ A, int lda,
                                                        const uint16_t *__restrict__ W,
                                                        const float *__restrict__ bias,
                                                        const float *res, void *out, int ldc,
                                                        int M, int N, int K) {
  constexpr int BK = 64, PITCH = BK + 8;
  constexpr int WM = BM / 2, WN = BN / 2, TM = WM / 32, TN = WN / 32;
  constexpr int CA = BM * BK / 8 / 256, CB = BN * BK / 8 / 256;  // 16-byte chunks per thread
  __shared__ __attribute__((aligned(16))) uint16_t sA[2][BM * PITCH];
  __shared__ __attribute__((aligned(16))) uint16_t sB[2][BN * PITCH];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t m0 = (int64_t)blockIdx.y * BM;
  const int n0 = blockIdx.x * BN;

  uint4 ra[CA], rb[CB];
  auto gload = [&](int k0) {
#pragma unroll
    for (int i = 0; i < CA; ++i) {
      const int c = tid + 256 * i, row = c >> 3, kc = c & 7;
      ra[i] = *reinterpret_cast<const uint4 *>(A + (m0 + row) * lda + k0 + kc * 8);
    }
#pragma unroll
    for (int i = 0; i < CB; ++i) {
      const int c = tid + 256 * i, row = c >> 3, kc = c & 7;
      rb[i] = *reinterpret_cast<const uint4 *>(W + (int64_t)(n0 + row) * K + k0 + kc * 8);
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < CA; ++i) {
      const int c = tid + 256 * i, row = c >> 3, kc = c & 7;
      *reinterpret_cast<uint4 *>(&sA[buf][row * PITCH + kc * 8]) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < CB; ++i) {
      const int c = tid + 256 * i, row = c >> 3, kc = c & 7;
      *reinterpret_cast<uint4 *>(&sB[buf][row * PITCH + kc * 8]) = rb[i];
    }
  };

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int nk = K / BK;
  gload(0);
  lstore(0);
  __syncthreads();
  const int fr = lane & 31, fk = (lane >> 5) * 8;  // fragment row and k offset of this lane
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) gload((kt + 1) * BK);
    const uint16_t *a_s = sA[cur] + (wm * WM + fr) * PITCH + fk;
    const uint16_t *b_s = sB[cur] + (wn * WN + fr) * PITCH + fk;
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      bf16x8 a[TM], b[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i)
        a[i] = *reinterpret_cast<const bf16x8 *>(a_s + i * 32 * PITCH + kk * 16);
#pragma unroll
      for (int j = 0; j < TN; ++j)
        b[j] = *reinterpret_cast<const bf16x8 *>(b_s + j * 32 * PITCH + kk * 16);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) lstore(cur ^ 1);
    __syncthreads();
  }

  // 32x32 accumulator layout: lane holds column (lane & 31); register r holds
  // row 8 * (r / 4) + 4 * (lane / 32) + (r % 4).
#pragma unroll
  for (int i = 0; i < TM; ++i) {
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int n = n0 + wn * WN + j * 32 + (lane & 31);
      if (n >= N) continue;
      const float bn = bias[n];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t m = m0 + wm * WM + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        if (m < M) epi_store<EPI>(out, res, ldc, m, n, acc[i][j][r] + bn);
      }
    }
  }
}

// ---------------------------------------------------------------- fp32 SIMT
// 64 x 64 tile, K step 16, 4 x 4 outputs per thread; for the fp32 model.
template <int EPI>
__global__ __launch_bounds__(256) void gemm_f32_kernel(const float *__restrict__ A, int lda,
                                                       const float *__restrict__ W,
                                                       const float *__restrict__ bias,
                                                       const float *res, float *out, int ldc,
                                                       int M, int N, int K) {
  constexpr int BT = 64, BK = 16;
  __shared__ float sA[BK][BT + 4], sB[BK][BT + 4];
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  const int64_t m0 = (int64_t)blockIdx.y * BT;
  const int n0 = blockIdx.x * BT;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < K; k0 += BK) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = tid + 256 * i, row = e >> 4, k = e & 15;
      sA[k][row] = A[(m0 + row) * lda + k0 + k];
      sB[k][row] = W[(int64_t)(n0 + row) * K + k0 + k];
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < BK; ++k) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = sA[k][ty + 16 * i];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = sB[k][tx + 16 * j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t m = m0 + ty + 16 * i;
    if (m >= M) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + tx + 16 * j;
      if (n >= N) continue;
      const float v = acc[i][j] + bias[n];
      if (EPI == kEpiBias || EPI == kEpiF32) out[m * ldc + n] = v;
      else if (EPI == kEpiGelu) out[m * ldc + n] = gelu_erf(v);
      else out[m * ldc + n] = v + res[m * ldc + n];
    }
  }
}

template <int BM, int BN>
hipError_t go_bf16(const uint16_t *A, int lda, const uint16_t *W, const float *bias,
                   const float *res, void *out, int ldc, int M, int N, int K, int epi,
                   hipStream_t st) {
  const dim3 grid((N + BN - 1) / BN, (M + BM - 1) / BM), block(256);
  switch (epi) {
    case kEpiBias:
      gemm_bf16_kernel<BM, BN, kEpiBias><<<grid, block, 0, st>>>(A, lda, W, bias, res, out, ldc, M, N, K);
      break;
    case kEpiGelu:
      gemm_bf16_kernel<BM, BN, kEpiGelu><<<grid, block, 0, st>>>(A, lda, W, bias, res, out, ldc, M, N, K);
      break;
    case kEpiResidual:
      gemm_bf16_kernel<BM, BN, kEpiResidual><<<grid, block, 0, st>>>(A, lda, W, bias, res, out, ldc, M, N, K);
      break;
    case kEpiF32:
      gemm_bf16_kernel<BM, BN, kEpiF32><<<grid, block, 0, st>>>(A, lda, W, bias, res, out, ldc, M, N, K);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

// Both tile shapes issue the same MFMA over K in the same order and K is never
// split, so each output's accumulation order does not depend on the tile
// chosen or on the other sequences in the batch.
hipError_t launch_gemm_bf16(const uint16_t *A, int lda, const uint16_t *W, const float *bias,
                            const float *res, void *out, int ldc, int M, int N, int K, int epi,
                            hipStream_t st) {
  if (M <= 0 || N <= 0) return hipSuccess;
  if (K <= 0 || K % 64) return hipErrorInvalidValue;
  const int64_t tiles_big = (int64_t)((M + 255) / 256) * ((N + 127) / 128);
  if (tiles_big >= 512) return go_bf16<256, 128>(A, lda, W, bias, res, out, ldc, M, N, K, epi, st);
  return go_bf16<128, 128>(A, lda, W, bias, res, out, ldc, M, N, K, epi, st);
}

hipError_t launch_gemm_f32(const float *A, int lda, const float *W, const float *bias,
                           const float *res, float *out, int ldc, int M, int N, int K, int epi,
                           hipStream_t st) {
  if (M <= 0 || N <= 0) return hipSuccess;
  if (K <= 0 || K % 16) return hipErrorInvalidValue;
  const dim3 grid((N + 63) / 64, (M + 63) / 64), block(256);
  switch (epi) {
    case kEpiBias: gemm_f32_kernel<kEpiBias><<<grid, block, 0, st>>>(A, lda, W, bias, res, out, ldc, M, N, K); break;
    case kEpiGelu: gemm_f32_kernel<kEpiGelu><<<grid, block, 0, st>>>(A, lda, W, bias, res, out, ldc, M, N, K); break;
    case kEpiResidual: gemm_f32_kernel<kEpiResidual><<<grid, block, 0, st>>>(A, lda, W, bias, res, out, ldc, M, N, K); break;
    case kEpiF32: gemm_f32_kernel<kEpiF32><<<grid, block, 0, st>>>(A, lda, W, bias, res, out, ldc, M, N, K); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace es
