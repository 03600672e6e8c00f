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
#include <cmath>

#include "device.h"
#include "kernels.h"

namespace es {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// One GEMM kernel instance: block tile BM x BN, K depth BK per pipeline
// stage, WGM x WGN wavefronts (each owning a (BM/WGM) x (BN/WGN) sub-tile of
// 32 x 32 MFMA tiles), PF register staging sets (global prefetch distance),
// MINW wavefronts per SIMD the register budget is set for.
template <int BM_, int BN_, int BK_, int WGM_, int WGN_, int PF_, int MINW_>
struct Cfg {
  static constexpr int BM = BM_, BN = BN_, BK = BK_, WGM = WGM_, WGN = WGN_, PF = PF_;
  static constexpr int MINW = MINW_;
  static constexpr int NT = 64 * WGM * WGN;
  static constexpr int WM = BM / WGM, WN = BN / WGN, TM = WM / 32, TN = WN / 32;
  static constexpr int CPR = BK / 8;            // 16-byte chunks per LDS row
  static constexpr int RPL = 256 / (BK * 2);    // rows sharing one 256-byte bank line
  static_assert(TM >= 1 && TN >= 1 && RPL >= 1, "bad tile");
  static_assert((BM * CPR) % NT == 0 && (BN * CPR) % NT == 0, "tile not divisible by threads");
};

// LDS tile layout: rows of BK bf16, no padding; the 16-byte k-chunks of row r
// are XOR-swizzled by (r / rows-per-line) mod chunks-per-row.  gfx950 LDS
// serves a 16-byte read for 16 lanes per cycle from 64 four-byte banks
// (256-byte lines), so the 16 rows read by 16 lanes at one k-chunk must land
// on 16 distinct (line offset, chunk slot) pairs -- they do (checked with
// SQ_LDS_BANK_CONFLICT = 0) -- while row-wise 16-byte writes stay contiguous.
template <class C>
__device__ __forceinline__ int swz_slot(int row, int chunk) {
  return chunk ^ ((row / C::RPL) % C::CPR);
}

// Staging registers of one stage: ROWS x BK bf16 spread over the block, 16
// bytes per thread per chunk, held in ONE vector value so it stays in VGPRs
// (an array here is demoted to scratch or LDS by the compiler).
template <class C, int ROWS>
struct Stage {
  static constexpr int N = ROWS * C::CPR / C::NT;
  typedef uint32_t vec_t __attribute__((ext_vector_type(4 * N)));
  vec_t v;
};

template <class C, int ROWS>
__device__ __forceinline__ void load_stage(Stage<C, ROWS> &r, const uint16_t *__restrict__ g,
                                           int64_t ld, int k0, int tid) {
#pragma unroll
  for (int i = 0; i < Stage<C, ROWS>::N; ++i) {
    const int c = tid + C::NT * i, row = c / C::CPR, kc = c % C::CPR;
    const uint4 u = *reinterpret_cast<const uint4 *>(g + row * ld + k0 + kc * 8);
    r.v[4 * i + 0] = u.x;
    r.v[4 * i + 1] = u.y;
    r.v[4 * i + 2] = u.z;
    r.v[4 * i + 3] = u.w;
  }
}

template <class C, int ROWS>
__device__ __forceinline__ void store_stage(const Stage<C, ROWS> &r, uint16_t *s, int tid) {
#pragma unroll
  for (int i = 0; i < Stage<C, ROWS>::N; ++i) {
    const int c = tid + C::NT * i, row = c / C::CPR, kc = c % C::CPR;
    *reinterpret_cast<uint4 *>(s + row * C::BK + (swz_slot<C>(row, kc) << 3)) =
        make_uint4(r.v[4 * i + 0], r.v[4 * i + 1], r.v[4 * i + 2], r.v[4 * i + 3]);
  }
}

// Four consecutive outputs (m, n..n+3) of one lane, with bias[n..n+3]
// already loaded in bv when n + 3 < N.
// With a residual, rv holds res[m][n..n+3], loaded ahead by the caller.
template <int EPI>
__device__ __forceinline__ void epi_store4_bias(void *out, const float *res, int ldc, int64_t m,
                                                int n, int N, float4 v, float4 bv, float4 rv,
                                                const float *__restrict__ bias) {
  const int64_t o = m * ldc + n;
  constexpr bool RES = EPI == kEpiResidual || EPI == kEpiResidualFfn;
  if (n + 3 < N) {
    v.x += bv.x; v.y += bv.y; v.z += bv.z; v.w += bv.w;
    if (EPI == kEpiBias || EPI == kEpiGelu) {
      if (EPI == kEpiGelu) {
        v.x = gelu_erf_bf16out(v.x); v.y = gelu_erf_bf16out(v.y);
        v.z = gelu_erf_bf16out(v.z); v.w = gelu_erf_bf16out(v.w);
      }
      *reinterpret_cast<uint2 *>(static_cast<uint16_t *>(out) + o) = make_uint2(f2bf2(v.x, v.y), f2bf2(v.z, v.w));
    } else {
      if (RES) {
        v.x += rv.x; v.y += rv.y; v.z += rv.z; v.w += rv.w;
      }
      *reinterpret_cast<float4 *>(static_cast<float *>(out) + o) = v;
    }
    return;
  }
  const float vv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    if (n + e >= N) break;
    float x = vv[e] + bias[n + e];
    if (EPI == kEpiBias) static_cast<uint16_t *>(out)[o + e] = f2bf(x);
    else if (EPI == kEpiGelu) static_cast<uint16_t *>(out)[o + e] = f2bf(gelu_erf_bf16out(x));
    else if (RES) static_cast<float *>(out)[o + e] = x + res[o + e];
    else static_cast<float *>(out)[o + e] = x;
  }
}

// Four consecutive outputs (m, n..n+3) of one lane.
template <int EPI>
__device__ __forceinline__ void epi_store4(void *out, const float *res, int ldc, int64_t m, int n,
                                           int N, float4 v, const float *__restrict__ bias) {
  const int64_t o = m * ldc + n;
  constexpr bool RES = EPI == kEpiResidual || EPI == kEpiResidualFfn;
  if (n + 3 < N) {
    const float4 b = *reinterpret_cast<const float4 *>(bias + n);
    v.x += b.x; v.y += b.y; v.z += b.z; v.w += b.w;
    if (EPI == kEpiBias || EPI == kEpiGelu) {
      if (EPI == kEpiGelu) {
        v.x = gelu_erf_bf16out(v.x); v.y = gelu_erf_bf16out(v.y);
        v.z = gelu_erf_bf16out(v.z); v.w = gelu_erf_bf16out(v.w);
      }
      uint2 u;
      u.x = f2bf2(v.x, v.y);
      u.y = f2bf2(v.z, v.w);
      *reinterpret_cast<uint2 *>(static_cast<uint16_t *>(out) + o) = u;
    } else {
      if (RES) {
        const float4 r = *reinterpret_cast<const float4 *>(res + o);
        v.x += r.x; v.y += r.y; v.z += r.z; v.w += r.w;
      }
      *reinterpret_cast<float4 *>(static_cast<float *>(out) + o) = v;
    }
    return;
  }
  const float vv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    if (n + e >= N) break;
    float x = vv[e] + bias[n + e];
    if (EPI == kEpiBias) static_cast<uint16_t *>(out)[o + e] = f2bf(x);
    else if (EPI == kEpiGelu) static_cast<uint16_t *>(out)[o + e] = f2bf(gelu_erf_bf16out(x));
    else if (RES) static_cast<float *>(out)[o + e] = x + res[o + e];
    else static_cast<float *>(out)[o + e] = x;
  }
}

// XCD-aware tile order: consecutive block ids go to different XCDs (8 of
// them), so remap them so each XCD works on a contiguous run of tiles, then
// walk the tiles in groups of 8 along one dimension, so the blocks resident
// on an XCD at one time share a few A row panels and weight tiles in its L2.
// Groups of 8 N-tiles (M advancing slowly) when such a group's weights are
// small (8 BN K bf16 <= 2 MiB) or cover all of N: then every weight tile is
// fetched about once per XCD and each A panel once per group; measured HBM
// reads per launch on the encoder's GEMMs drop 3-34 % against groups of 8
// M-tiles (FFN1 126 -> 112 MB at M ~ 14.6k).  Otherwise (the decoder's wide,
// long-K weights) groups of 8 M-tiles, which re-read the weight panel once
// per group instead of re-reading the much larger A rows.
__device__ __forceinline__ void tile_of_block(int tiles_m, int tiles_n, int64_t w_group_bytes,
                                              int &tm, int &tn) {
  const int bid = xcd_contiguous(blockIdx.x, tiles_m * tiles_n);
  constexpr int G = 8;
  if (tiles_n <= G || w_group_bytes <= ((int64_t)2 << 20)) {
    const int group = bid / (G * tiles_m), first_n = group * G;
    const int gn = min(G, tiles_n - first_n);
    tn = first_n + (bid % (G * tiles_m)) % gn;
    tm = (bid % (G * tiles_m)) / gn;
  } else {
    const int group = bid / (G * tiles_n), first_m = group * G;
    const int gm = min(G, tiles_m - first_m);
    tm = first_m + (bid % (G * tiles_n)) % gm;
    tn = (bid % (G * tiles_n)) / gm;
  }
}

// ---------------------------------------------------------------- bf16 MFMA
//
// A and W tiles stage through two LDS buffers; with PF = 2 they are fed from
// two register staging sets so the global loads of step k+2 are in flight
// while the matrix cores work on step k (PF = 1: loads of step k+1).  One
// barrier per step.  The MFMA is issued as W x A so a lane's accumulators hold
// four consecutive output columns of one row, which the epilogue writes as
// one vector.
template <class C, int EPI>
__global__ __launch_bounds__(C::NT, C::MINW) void gemm_bf16_kernel(
    const uint16_t *__restrict__ A, int lda, const uint16_t *__restrict__ W,
    const float *__restrict__ bias, const float *res, void *out, int ldc, int M, int N, int K,
    int tiles_m, int tiles_n) {
  constexpr int BM = C::BM, BN = C::BN, BK = C::BK, TM = C::TM, TN = C::TN;
  __shared__ __attribute__((aligned(16))) uint16_t sA[2][BM * BK];
  __shared__ __attribute__((aligned(16))) uint16_t sB[2][BN * BK];

  int tm, tn;
  tile_of_block(tiles_m, tiles_n, (int64_t)8 * C::BN * K * 2, tm, tn);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / C::WGN, wn = wave % C::WGN;
  const int64_t m0 = (int64_t)tm * BM;
  const int n0 = tn * BN;
  const uint16_t *Ag = A + m0 * lda;
  const uint16_t *Wg = W + (int64_t)n0 * K;

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int fr = lane & 31, fh = lane >> 5;  // fragment row, k-half of this lane
  const uint16_t *a_base = sA[0] + (C::WM * wm + fr) * BK;
  const uint16_t *b_base = sB[0] + (C::WN * wn + fr) * BK;
  auto mma_tile = [&](int buf) {
    const uint16_t *a_s = a_base + buf * BM * BK;
    const uint16_t *b_s = b_base + buf * BN * BK;
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      const int slot = swz_slot<C>(fr, kk * 2 + fh) << 3;
      bf16x8 a[TM], b[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i)
        a[i] = *reinterpret_cast<const bf16x8 *>(a_s + i * 32 * BK + slot);
#pragma unroll
      for (int j = 0; j < TN; ++j)
        b[j] = *reinterpret_cast<const bf16x8 *>(b_s + j * 32 * BK + slot);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b[j], a[i], acc[i][j], 0, 0, 0);
    }
  };

  const int nk = K / BK;
  Stage<C, BM> ra0, ra1;
  Stage<C, BN> rb0, rb1;
  load_stage<C, BM>(ra0, Ag, lda, 0, tid);
  load_stage<C, BN>(rb0, Wg, K, 0, tid);
  if (C::PF == 2) {  // tile 1 (tile 0 again when K has one step: see below)
    load_stage<C, BM>(ra1, Ag, lda, min(1, nk - 1) * BK, tid);
    load_stage<C, BN>(rb1, Wg, K, min(1, nk - 1) * BK, tid);
  }
  store_stage<C, BM>(ra0, sA[0], tid);
  store_stage<C, BN>(rb0, sB[0], tid);
  __syncthreads();

  if (C::PF == 2) {
    // LDS buffer kt & 1 holds tile kt, register set (kt + 1) & 1 holds tile
    // kt + 1, loads of tile kt + 2 go into the free set.  Unrolled by two so
    // both register sets are fixed names.  The loads are issued on every
    // step, past the end at tile nk - 1 again (in bounds, never stored): a
    // load under a branch makes the compiler's wait before the next LDS
    // store drain every load in flight, which left one step of prefetch.
    for (int kt = 0; kt < nk; kt += 2) {
      load_stage<C, BM>(ra0, Ag, lda, min(kt + 2, nk - 1) * BK, tid);
      load_stage<C, BN>(rb0, Wg, K, min(kt + 2, nk - 1) * BK, tid);
      mma_tile(0);
      if (kt + 1 < nk) {
        store_stage<C, BM>(ra1, sA[1], tid);
        store_stage<C, BN>(rb1, sB[1], tid);
      }
      __syncthreads();
      if (kt + 1 >= nk) break;
      load_stage<C, BM>(ra1, Ag, lda, min(kt + 3, nk - 1) * BK, tid);
      load_stage<C, BN>(rb1, Wg, K, min(kt + 3, nk - 1) * BK, tid);
      mma_tile(1);
      if (kt + 2 < nk) {
        store_stage<C, BM>(ra0, sA[0], tid);
        store_stage<C, BN>(rb0, sB[0], tid);
      }
      __syncthreads();
    }
  } else {
    for (int kt = 0; kt < nk; ++kt) {
      const int cur = kt & 1;
      const bool more = kt + 1 < nk;
      if (more) {
        load_stage<C, BM>(ra0, Ag, lda, (kt + 1) * BK, tid);
        load_stage<C, BN>(rb0, Wg, K, (kt + 1) * BK, tid);
      }
      mma_tile(cur);
      if (more) {
        store_stage<C, BM>(ra0, sA[cur ^ 1], tid);
        store_stage<C, BN>(rb0, sB[cur ^ 1], tid);
      }
      __syncthreads();
    }
  }

  // acc[i][j] = D[n][m] of the W x A product: lane holds row m = lane & 31
  // and register r holds column 8 * (r / 4) + 4 * (lane / 32) + (r % 4).
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    const int64_t m = m0 + C::WM * wm + i * 32 + fr;
    if (m >= M) continue;
#pragma unroll
    for (int j = 0; j < TN; ++j) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int n = n0 + C::WN * wn + j * 32 + 8 * g + 4 * fh;
        if (n < N)
          epi_store4<EPI>(out, res, ldc, m, n, N,
                          make_float4(acc[i][j][4 * g], acc[i][j][4 * g + 1],
                                      acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]),
                          bias);
      }
    }
  }
}

// ---------------------------------------------------------------- bf16 MFMA, ping-pong
//
// Block BM x BN x 64, eight wavefronts in two groups of four (wave w runs on
// SIMD w % 4, so each SIMD holds one wave of each group).  Group g owns the
// output rows [g BM/2, (g+1) BM/2); wave q of a group owns the columns
// [q BN/4, (q+1) BN/4).  The groups alternate between two phases that a
// barrier separates: in one a wave reads a whole K stage of fragments from
// LDS into registers, in the other it runs that stage's MFMAs back to back.
// Group 1 runs one phase behind group 0, so on every SIMD one wave keeps the
// matrix core busy while the other reads LDS, and no barrier leaves a SIMD
// without MFMA work.
//
// Stages reach LDS by direct loads (buffer_load ... lds: L2 to LDS without
// VGPRs) issued by group 0 one stage ahead into the buffer group 1 has just
// finished reading; two 64-deep stage buffers.  A stage's rows are written
// in the swizzled layout above by permuting, per lane, which 16-byte chunk of
// the row it fetches.
typedef int i32x4 __attribute__((ext_vector_type(4)));

// 16 bytes per lane from a buffer resource into LDS at lds + 16 * lane.  The
// load is inline asm because the compiler's wait-count pass, when it sees
// direct-to-LDS loads in a loop, waits for all of them before every LDS read;
// the kernels order these loads with explicit vmcnt waits and barriers.  M0
// (the LDS base of the load) is saved and restored within the statement, and
// one wait state separates the M0 write from the load that reads it.
__device__ __forceinline__ void dma16(i32x4 rsrc, int voff, int soff, uint32_t lds) {
  int saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %4\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %1, %2, %3 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(voff), "s"(rsrc), "s"(soff), "s"(lds)
      : "memory");
}

// 4 bytes per lane into LDS at lds + 4 * lane: used only to pull lines of a
// later stage into L2 ahead of its real load (the LDS words are never read).
__device__ __forceinline__ void dma4(i32x4 rsrc, int voff, int soff, uint32_t lds) {
  int saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %4\n\t"
      "s_nop 0\n\t"
      "buffer_load_dword %1, %2, %3 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(voff), "s"(rsrc), "s"(soff), "s"(lds)
      : "memory");
}

// Raw buffer resource over [p, p + 2 GB): base, stride 0, num_records,
// 32-bit dword format.
__device__ __forceinline__ i32x4 make_rsrc(const void *p) {
  const uint64_t a = (uint64_t)p;
  i32x4 r;
  r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  r[1] = __builtin_amdgcn_readfirstlane((int)((uint32_t)(a >> 32) & 0xffff));
  r[2] = 0x7ffffff0;
  r[3] = 0x00020000;
  return r;
}

__device__ __forceinline__ uint32_t lds_addr(const void *p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)p;
}

// vmcnt(n) and lgkmcnt(0) in one s_waitcnt; lgkmcnt(0) alone.
__device__ __forceinline__ constexpr int wait_vm_lgkm0(int n) {
  return (n & 15) | ((n >> 4) << 14) | (7 << 4);
}
constexpr int kWaitLgkm0 = 0xc07f;

template <int BM_, int BN_>
struct PPCfg {
  static constexpr int BM = BM_, BN = BN_, BK = 64;
  static constexpr int WM = BM / 2, WN = BN / 4, TM = WM / 32, TN = WN / 32;
  static constexpr int CPR = BK / 8, RPL = 256 / (BK * 2), KS = BK / 16;
  static constexpr int NL = 4;  // wavefronts issuing the direct loads (group 0)
  static constexpr int NIA = BM * CPR / (64 * NL), NIB = BN * CPR / (64 * NL);
  static constexpr int SZ = (BM + BN) * BK;  // bf16 elements per stage
  // rows between consecutive loads of one wave; the swizzle repeats every
  // such step, so one per-lane offset serves all of a wave's loads
  static constexpr int DR = NL * 64 / CPR;
  static_assert(TM >= 1 && TN >= 1, "bad tile");
  static_assert(NIA * 64 * NL == BM * CPR && NIB * 64 * NL == BN * CPR, "stage not divisible");
  static_assert(DR % RPL == 0 && (DR / RPL) % CPR == 0, "swizzle must repeat between loads");
};

// Staged epilogue of the eight-wavefront blocks (wave (grp, q) owns rows
// [grp WM, (grp+1) WM) and columns [q WN, (q+1) WN) of the block).
// acc[i][j] = D[n][m] of the W x A product: lane holds row m = lane & 31 and
// register r column 8 (r / 4) + 4 (lane / 32) + (r % 4), so stored straight
// from registers one instruction writes 16-32 bytes in each of 32 rows.
// Instead each wave stages 32 rows of its accumulators at a time in its own
// LDS region of `buf` (a stage buffer, free once the K loop is done) and
// reads them back along rows: a lane then owns one 4-column chunk, bias (and
// residual) loads and output stores cover whole row segments.  Rows are
// padded by 4 floats so both the staging writes and the row reads spread
// over the LDS banks.  Every access is by the wave that wrote it and a
// wave's LDS operations execute in program order, so no barrier is needed;
// wavefront-scope fences (no instructions) keep the compiler from moving a
// lane's reads of other lanes' writes across them.
template <class C, int EPI>
__device__ __forceinline__ void staged_epilogue(const f32x16 (&acc)[C::TM][C::TN], float *buf, int grp,
                                                int q, int lane, int64_t m0, int n0,
                                                const float *__restrict__ bias, const float *res,
                                                void *out, int ldc, int M, int N) {
  constexpr int TM = C::TM, TN = C::TN;
  const int fr = lane & 31, fh = lane >> 5;
  constexpr int PITCH = C::WN + 4;              // floats per staged row
  constexpr int CH = C::WN / 4;                 // 4-column chunks per row
  constexpr int RPI = 64 / CH;                  // rows per read instruction (lanes beyond
                                                // RPI * CH idle when CH does not divide 64)
  static_assert(4 * 32 * PITCH * 4 <= C::SZ * 2, "epilogue staging exceeds a stage buffer");
  float *stage = buf + q * 32 * PITCH;  // group g in buffer g
  const int cc = lane % CH, rr = lane / CH;
  const int n = n0 + C::WN * q + 4 * cc;
  float4 bv = make_float4(0.f, 0.f, 0.f, 0.f);
  if (n + 3 < N) bv = *reinterpret_cast<const float4 *>(bias + n);
  constexpr bool RES = EPI == kEpiResidual || EPI == kEpiResidualFfn;
  constexpr int NR = (32 + RPI - 1) / RPI;      // row reads per 32-row slab
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    // the slab's residual chunks, all issued before the first is used (one
    // memory round trip per slab, not one per row read); indices clamped
    // into the output's rows and columns, rows or chunks outside it are
    // never stored (N < 4 takes the per-element path, which reads res itself)
    float4 rv[NR];
#pragma unroll
    for (int k = 0; k < NR; ++k) rv[k] = make_float4(0.f, 0.f, 0.f, 0.f);
    if (RES && N >= 4) {
#pragma unroll
      for (int k = 0; k < NR; ++k) {
        const int64_t m = min(m0 + C::WM * grp + i * 32 + k * RPI + rr, (int64_t)M - 1);
        rv[k] = *reinterpret_cast<const float4 *>(res + m * ldc + min(n, N - 4));
      }
    }
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        *reinterpret_cast<float4 *>(stage + fr * PITCH + j * 32 + 8 * g + 4 * fh) =
            make_float4(acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]);
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
#pragma unroll
    for (int k = 0; k < NR; ++k) {
      const int row = k * RPI + rr;
      if (rr < RPI && row < 32) {
        const int64_t m = m0 + C::WM * grp + i * 32 + row;
        const float4 v = *reinterpret_cast<const float4 *>(stage + row * PITCH + 4 * cc);
        if (m < M && n < N) epi_store4_bias<EPI>(out, res, ldc, m, n, N, v, bv, rv[k], bias);
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
  }
}

template <class C, int EPI, int PFD>
__global__ __launch_bounds__(512, 2) void gemm_pp_kernel(
    const uint16_t *__restrict__ A, int lda, const uint16_t *__restrict__ W,
    const float *__restrict__ bias, const float *res, void *out, int ldc, int M, int N, int K,
    int tiles_m, int tiles_n) {
  constexpr int BM = C::BM, BK = C::BK, TM = C::TM, TN = C::TN, KS = C::KS, DR = C::DR;
  // two named buffers (not one array) so the compiler can tell their
  // accesses apart
  __shared__ __attribute__((aligned(1024))) uint16_t L0[C::SZ];
  __shared__ __attribute__((aligned(1024))) uint16_t L1[C::SZ];
  __shared__ uint32_t Lpf[64];  // landing words of the L2 prefetches (never read)

  int tm, tn;
  tile_of_block(tiles_m, tiles_n, (int64_t)8 * C::BN * K * 2, tm, tn);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2, q = wave & 3;
  const int64_t m0 = (int64_t)tm * BM;
  const int n0 = tn * C::BN;
  const uint16_t *Ag = A + m0 * lda;
  const uint16_t *Wg = W + (int64_t)n0 * K;

  const i32x4 ra = make_rsrc(Ag), rb = make_rsrc(Wg);
  int voA, voB;  // byte offsets of this lane's chunk in the wave's first load
  {
    const int e = q * 64 + lane, row = e / C::CPR, slot = e % C::CPR;
    voA = (row * lda + swz_slot<C>(row, slot) * 8) * 2;
    voB = (row * K + swz_slot<C>(row, slot) * 8) * 2;
  }
  auto issue = [&](uint16_t *buf, int k0) {
    const uint32_t l0 = lds_addr(buf) + q * 1024;
#pragma unroll
    for (int i = 0; i < C::NIA; ++i) dma16(ra, voA, (k0 + i * DR * lda) * 2, l0 + i * C::NL * 1024);
#pragma unroll
    for (int i = 0; i < C::NIB; ++i)
      dma16(rb, voB, (k0 + i * DR * K) * 2, l0 + BM * BK * 2 + i * C::NL * 1024);
  };
  // With PFD > 0, group 0 also touches every 32-byte sector of the A panel of
  // stage k + 1 + PFD right after issuing stage k + 1, so that stage's real
  // loads find it in L2 instead of waiting on HBM: A is the operand streamed
  // from memory (W is shared by every block and stays in L2).  One 4-byte
  // load per sector; lane e of the group covers row e / 4, sector e % 4.
  constexpr int NPA = BM * 4 / (64 * C::NL);
  const int voP = ((q * 64 + lane) / 4 * lda + (lane % 4) * 16) * 2;
  auto prefetch = [&](int k0) {
    const uint32_t lp = lds_addr(Lpf);
#pragma unroll
    for (int i = 0; i < NPA; ++i) dma4(ra, voP, (k0 + i * 64 * lda) * 2, lp);
  };

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int fr = lane & 31, fh = lane >> 5;
  bf16x8 fa[KS][TM], fb[KS][TN];
  auto read_stage = [&](const uint16_t *buf) {
    const uint16_t *a_s = buf + (C::WM * grp + fr) * BK;
    const uint16_t *b_s = buf + BM * BK + (C::WN * q + fr) * BK;
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      const int slot = swz_slot<C>(fr, kk * 2 + fh) << 3;
#pragma unroll
      for (int i = 0; i < TM; ++i) fa[kk][i] = *reinterpret_cast<const bf16x8 *>(a_s + i * 32 * BK + slot);
#pragma unroll
      for (int j = 0; j < TN; ++j) fb[kk][j] = *reinterpret_cast<const bf16x8 *>(b_s + j * 32 * BK + slot);
    }
  };
  auto mma_stage = [&]() {
#pragma unroll
    for (int kk = 0; kk < KS; ++kk)
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[kk][j], fa[kk][i], acc[i][j], 0, 0, 0);
  };
  // Nothing is scheduled across a phase boundary: the compiler would
  // otherwise move MFMAs over the barrier and merge the two phases.
  // wait_loads: 0 none, 1 all loads, 2 all but the prefetches issued last.
  auto end_phase = [&](int wait_loads) {
    __builtin_amdgcn_sched_barrier(0);
    if (wait_loads == 2) __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0(NPA));
    else if (wait_loads == 1) __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0(0));
    else __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
  };

  // Phase p lies between barriers p and p+1.  Group 0 reads stage k in phase
  // 2k and computes it in phase 2k+1; group 1 one phase later.  Group 0
  // issues stage k+1 at the start of phase 2k into the buffer that group 1
  // finished reading in phase 2k-1, and waits for it at the end of phase
  // 2k+1, before it reads it.  Both groups pass 2 nk + 2 barriers.
  //
  // Prefetches: stages 1 .. PFD before the loop, stage k + 1 + PFD after
  // stage k + 1's loads.  Loads complete in order, so the wait at the end of
  // phase 2k+1 may leave that last batch of prefetches in flight.
  const int nk = K / BK;
  if (grp == 0) {
    issue(L0, 0);
    if (PFD > 0)
      for (int p = 1; p <= PFD && p < nk; ++p) prefetch(p * BK);
    __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0(0));
  }
  __builtin_amdgcn_s_barrier();
  if (grp == 1) __builtin_amdgcn_s_barrier();
  for (int k0 = 0; k0 < nk; k0 += 2) {
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int k = k0 + s;
      if (k < nk) {
        uint16_t *cur = s == 0 ? L0 : L1;
        uint16_t *nxt = s == 0 ? L1 : L0;
        const bool pf = PFD > 0 && k + 1 + PFD < nk;
        if (grp == 0 && k + 1 < nk) {
          issue(nxt, (k + 1) * BK);
          if (pf) prefetch((k + 1 + PFD) * BK);
        }
        read_stage(cur);
        end_phase(0);
        mma_stage();
        end_phase(grp == 0 ? (pf ? 2 : 1) : 0);
      }
    }
  }
  if (grp == 0) __builtin_amdgcn_s_barrier();

  staged_epilogue<C, EPI>(acc, reinterpret_cast<float *>(grp == 0 ? L0 : L1), grp, q, lane, m0, n0,
                          bias, res, out, ldc, M, N);
}

// ---------------------------------------------------------------- bf16 MFMA, software pipeline
//
// Block BM x BN x 64 with the eight-wavefront layout of the ping-pong blocks
// (wave (grp, q) owns a WM x WN sub-tile), but every wavefront runs the same
// schedule, pipelined one MFMA k-step (16 deep) ahead: while the matrix core
// works through a k-step's TM x TN MFMAs, the LDS reads of the next k-step's
// fragments are in flight.  Scheduling fences pin that order (left alone,
// the compiler issues the reads after the MFMAs that free their registers
// and waits for them at once).  All eight wavefronts share the direct loads;
// one barrier per stage, after the last k-step's reads, with this
// wavefront's loads of the next stage landed first.  Two waves per SIMD
// interleave their MFMA streams, so neither the barrier nor the LDS latency
// leaves the matrix core idle for long.
//
// A (the activations, streamed from HBM when the pass is large) has NA stage
// buffers and W (the weights, mostly L2 hits) two: stage k + NA - 1's A
// loads go out during stage k, so they have NA - 1 stages to arrive; stage
// k + 1's W loads go out at the start of stage k.  With NA = 3 and a 256 x
// 256 block that is the whole 160 KiB of LDS.
template <int BM_, int BN_, int NA_>
struct SPCfg {
  static constexpr int BM = BM_, BN = BN_, BK = 64, NA = NA_;
  static constexpr int WM = BM / 2, WN = BN / 4, TM = WM / 32, TN = WN / 32;
  static constexpr int CPR = BK / 8, RPL = 256 / (BK * 2), KS = BK / 16;
  static constexpr int NL = 8;  // wavefronts issuing the direct loads (all)
  static constexpr int NIA = BM * CPR / (64 * NL), NIB = BN * CPR / (64 * NL);
  static constexpr int ABYTES = BM * BK * 2, BBYTES = BN * BK * 2;  // one stage of A / of W
  static constexpr int LDS = NA * ABYTES + 2 * BBYTES;
  static constexpr int SZ = (BM + BN) * BK;  // bf16 elements of an A + W stage (epilogue regions)
  static constexpr int DR = NL * 64 / CPR;
  static_assert(TM >= 1 && TN >= 1 && NA >= 2, "bad tile");
  static_assert(NIA * 64 * NL == BM * CPR && NIB * 64 * NL == BN * CPR, "stage not divisible");
  static_assert(DR % RPL == 0 && (DR / RPL) % CPR == 0, "swizzle must repeat between loads");
  static_assert(LDS <= 160 * 1024 && 2 * SZ * 2 <= LDS, "LDS budget");
};

template <class C, int EPI>
__global__ __launch_bounds__(512, 1) void gemm_sp_kernel(
    const uint16_t *__restrict__ A, int lda, const uint16_t *__restrict__ W,
    const float *__restrict__ bias, const float *res, void *out, int ldc, int M, int N, int K,
    int tiles_m, int tiles_n) {
  constexpr int BM = C::BM, BK = C::BK, TM = C::TM, TN = C::TN, KS = C::KS, DR = C::DR, NA = C::NA;
  // A stage buffers at [0, NA ABYTES), W stage buffers after them
  __shared__ __attribute__((aligned(1024))) uint8_t lds[C::LDS];

  int tm, tn;
  tile_of_block(tiles_m, tiles_n, (int64_t)8 * C::BN * K * 2, tm, tn);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2, q = wave & 3;
  const int64_t m0 = (int64_t)tm * BM;
  const int n0 = tn * C::BN;
  const uint16_t *Ag = A + m0 * lda;
  const uint16_t *Wg = W + (int64_t)n0 * K;

  const i32x4 ra = make_rsrc(Ag), rb = make_rsrc(Wg);
  int voA, voB;  // byte offsets of this lane's chunk in the wave's first load
  {
    const int e = wave * 64 + lane, row = e / C::CPR, slot = e % C::CPR;
    voA = (row * lda + swz_slot<C>(row, slot) * 8) * 2;
    voB = (row * K + swz_slot<C>(row, slot) * 8) * 2;
  }
  const uint32_t lds0 = lds_addr(lds);
  // this wavefront's direct loads of one stage of A / of W, each chunk
  // landing at its swizzled LDS position
  auto issue_a = [&](int stage) {
    const uint32_t l0 = lds0 + (stage % NA) * C::ABYTES + wave * 1024;
    const int k0 = stage * BK;
#pragma unroll
    for (int t = 0; t < C::NIA; ++t) dma16(ra, voA, (k0 + t * DR * lda) * 2, l0 + t * C::NL * 1024);
  };
  auto issue_b = [&](int stage) {
    const uint32_t l0 = lds0 + NA * C::ABYTES + (stage & 1) * C::BBYTES + wave * 1024;
    const int k0 = stage * BK;
#pragma unroll
    for (int t = 0; t < C::NIB; ++t) dma16(rb, voB, (k0 + t * DR * K) * 2, l0 + t * C::NL * 1024);
  };

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int fr = lane & 31, fh = lane >> 5;
  const uint16_t *a_lane = reinterpret_cast<const uint16_t *>(lds) + (C::WM * grp + fr) * BK;
  const uint16_t *b_lane =
      reinterpret_cast<const uint16_t *>(lds + NA * C::ABYTES) + (C::WN * q + fr) * BK;
  bf16x8 fa[2][TM], fb[2][TN];
  auto read_kstep = [&](int set, int stage, int kk) {
    const uint16_t *a_s = a_lane + (stage % NA) * (C::ABYTES / 2);
    const uint16_t *b_s = b_lane + (stage & 1) * (C::BBYTES / 2);
    const int slot = swz_slot<C>(fr, kk * 2 + fh) << 3;
#pragma unroll
    for (int i = 0; i < TM; ++i) fa[set][i] = *reinterpret_cast<const bf16x8 *>(a_s + i * 32 * BK + slot);
#pragma unroll
    for (int j = 0; j < TN; ++j) fb[set][j] = *reinterpret_cast<const bf16x8 *>(b_s + j * 32 * BK + slot);
  };
  auto mma_kstep = [&](int set) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[set][j], fa[set][i], acc[i][j], 0, 0, 0);
  };

  const int nk = K / BK;
  // prologue: A stages 0 .. NA - 2 and W stage 0; wait for stage 0 only
  // (loads complete in order)
  issue_a(0);
  issue_b(0);
  for (int p = 1; p < NA - 1; ++p)
    if (p < nk) issue_a(p);
  {
    const int ahead = min(NA - 2, nk - 1);  // A stages issued after W stage 0
    if (ahead >= 2) __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0(2 * C::NIA));
    else if (ahead == 1) __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0(C::NIA));
    else __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0(0));
  }
  __builtin_amdgcn_s_barrier();
  read_kstep(0, 0, 0);
  __builtin_amdgcn_sched_barrier(0);

  // Stage k: k-step kk computes on fragment set kk & 1 (read one k-step
  // earlier) while the next k-step's reads fly.  W stage k + 1 goes out in
  // k-step 0 and A stage k + NA - 1 in k-step 1, into buffers whose last
  // reads (stage k - 1) every wavefront finished before the previous
  // barrier.  The last k-step waits for A and W stage k + 1 (leaving A stage
  // k + NA - 1 in flight) and for its LDS reads, passes the barrier, then
  // reads stage k + 1's first fragments.
  for (int k = 0; k < nk; ++k) {
    const bool more = k + 1 < nk;
    const bool far = k + NA - 1 < nk;
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      const int set = kk & 1;
      if (kk + 1 < KS) {
        read_kstep(set ^ 1, k, kk + 1);
        if (kk == 0 && more) issue_b(k + 1);
        if (kk == 1 && far) issue_a(k + NA - 1);
      } else {
        if (NA > 2 && far) __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0(C::NIA));
        else __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0(0));
        __builtin_amdgcn_s_barrier();
        if (more) read_kstep(set ^ 1, k + 1, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
      mma_kstep(set);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  // every wavefront's last fragment reads completed before the final
  // barrier, so the whole LDS is free for the staging
  staged_epilogue<C, EPI>(acc, reinterpret_cast<float *>(lds + grp * C::SZ * 2), grp, q, lane, m0,
                          n0, bias, res, out, ldc, M, N);
}

// ------------------------------------------------------ split-precision tile
// out = epi(A W^T + bias) for fp32 activations A against the bf16 weights, on
// bf16 MFMA with fp32 accumulation: each A element enters as the pair hi =
// bf16(a), lo = bf16(a - hi), two MFMAs per k-step into one accumulator, so
// the operand keeps 16 significant bits (|a - hi - lo| <= 2^-16 |a|) instead
// of bf16's 8.  It serves the last-token refinement of the reward rows: one
// row per sequence, fp32 throughout, so those rows carry none of the bulk
// path's bf16 activation rounding.  A arrives already split, in fragment
// order (split_off): each of its loads is 1 KB of contiguous memory per
// wavefront, where fp32 rows read straight into the fragments touched 32
// cache lines per load and ran at half the speed.  Few rows, so the weights
// dominate the bytes: one block of KW wavefronts per 32 output columns and
// MT 32-row tiles, each W fragment loaded once for all MT row tiles;
// wavefront w takes the w-th of KW equal k-ranges, operands loaded straight
// into registers D k-steps ahead (the latency tile's fragment layout), and
// the KW partial tiles are summed in wavefront order through LDS.  W rows
// past N are read at the last row and never stored.  Epilogues: kEpiF32
// acc + bias and kEpiResidual acc + bias + res[m, n] (res may be out) into
// fp32 rows; kEpiGelu GELU(acc + bias) (device erff) into outp, split again
// (split_off with K' = N) for the next split GEMM.
template <int EPI, int MT, int D>
__global__ __launch_bounds__(256) void gemm_split_kernel(const uint16_t *__restrict__ A,
                                                         const uint16_t *__restrict__ W,
                                                         const float *__restrict__ bias,
                                                         const float *res, float *out,
                                                         uint16_t *__restrict__ outp, int ldc, int M,
                                                         int N, int K, int tiles_n) {
  __shared__ __align__(16) float part[3][MT][16][64];
  const int lane = threadIdx.x % 64, wv = threadIdx.x / 64, kw = blockDim.x / 64;
  const int fr = lane & 31, fh = lane >> 5;
  const int ch = blockIdx.x / tiles_n, tn = blockIdx.x % tiles_n;
  const int mtiles = (M + 31) / 32;
  const int nkt = K / 16, nk = nkt / kw, kb = wv * nk;  // this wavefront's k-steps [kb, kb + nk)
  const int n0 = tn * 32;
  const uint16_t *ap[MT];  // k-step k of row tile t: hi at ap[t] + 1024 k, lo 512 further
#pragma unroll
  for (int t = 0; t < MT; ++t)
    ap[t] = A + (((int64_t)min(ch * MT + t, mtiles - 1) * nkt + kb) * 128 + lane) * 8;
  const uint16_t *wp = W + (int64_t)min(n0 + fr, N - 1) * K + 8 * fh + 16 * kb;
  static_assert(D % 4 == 0, "the tail runs in groups of 4 k-steps");
  bf16x8 fa[D][MT][2], fb[D];
  auto load = [&](int d, int k) {
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      fa[d][t][0] = *reinterpret_cast<const bf16x8 *>(ap[t] + 1024 * k);
      fa[d][t][1] = *reinterpret_cast<const bf16x8 *>(ap[t] + 1024 * k + 512);
    }
    fb[d] = *reinterpret_cast<const bf16x8 *>(wp + 16 * k);
  };
#pragma unroll
  for (int d = 0; d < D; ++d) load(d, min(d, nk - 1));
  f32x16 acc[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[t][r] = 0.f;
  auto mma = [&](int d) {
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[d], fa[d][t][0], acc[t], 0, 0, 0);
      acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[d], fa[d][t][1], acc[t], 0, 0, 0);
    }
  };
  int k = 0;
  for (; k + D <= nk; k += D) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      mma(d);
      load(d, min(k + d + D, nk - 1));
      __builtin_amdgcn_sched_barrier(0);
    }
  }
#pragma unroll
  for (int d = 0; d < D; d += 4) {
    if (k + d < nk) {
#pragma unroll
      for (int e = 0; e < 4; ++e) mma(d + e);
    }
  }
  if (wv > 0) {
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) part[wv - 1][t][r][lane] = acc[t][r];
  }
  __syncthreads();
  if (wv > 0) return;
  for (int w = 1; w < kw; ++w) {
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[t][r] += part[w - 1][t][r][lane];
  }
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    const int64_t m = (int64_t)(ch * MT + t) * 32 + fr;
    if (m >= M) break;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int n = n0 + 8 * g + 4 * fh;
      if (EPI == kEpiGelu) {  // N a multiple of 16: all four or none
        if (n >= N) break;
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = gelu_erf(acc[t][4 * g + e] + bias[n + e]);
        uint2 hi, lo;
        split4(v, hi, lo);
        *reinterpret_cast<uint2 *>(outp + split_off(m, n, N, 0)) = hi;
        *reinterpret_cast<uint2 *>(outp + split_off(m, n, N, 1)) = lo;
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if (n + e >= N) break;
          float x = acc[t][4 * g + e] + bias[n + e];
          if (EPI == kEpiResidual) x += res[m * ldc + n + e];
          out[m * ldc + n + e] = x;
        }
      }
    }
  }
}

// ------------------------------------------------------------ latency tile
// One wavefront per 32 x 32 output tile, operands loaded from global memory
// straight into the MFMA's registers, D k-steps of 16 ahead: no LDS and no
// barrier.  Lane (r, h) loads, for k-step kk, the 16-byte chunk of row r at
// columns 16 kk + 8 h .. + 8 of A and of W -- the fragment the LDS-staged
// blocks hand to the same MFMA -- so each output accumulates bitwise as in
// every other tile.  For the small passes (one short sequence, a last layer
// pruned to one row per sequence) a block's time is the chain of K / 16
// dependent MFMAs plus memory latency; the LDS-staged blocks add an LDS
// write, a barrier and an LDS read round trip to every k-step of that chain.
template <int EPI, int D>
__global__ __launch_bounds__(64) void gemm_lat_kernel(const uint16_t *__restrict__ A, int lda,
                                                      const uint16_t *__restrict__ W,
                                                      const float *__restrict__ bias,
                                                      const float *res, void *out, int ldc, int M,
                                                      int N, int K, int tiles_n) {
  const int lane = threadIdx.x, fr = lane & 31, fh = lane >> 5;
  const int tm = blockIdx.x / tiles_n, tn = blockIdx.x % tiles_n;
  const int64_t m0 = (int64_t)tm * 32;
  const int n0 = tn * 32;
  const uint16_t *ap = A + (m0 + fr) * lda + 8 * fh;
  const uint16_t *wp = W + (int64_t)(n0 + fr) * K + 8 * fh;
  const int nk = K / 16;
  static_assert(D % 4 == 0, "the tail runs in groups of 4 k-steps");
  bf16x8 fa[D], fb[D];
#pragma unroll
  for (int d = 0; d < D; ++d) {
    const int k = min(d, nk - 1);
    fa[d] = *reinterpret_cast<const bf16x8 *>(ap + 16 * k);
    fb[d] = *reinterpret_cast<const bf16x8 *>(wp + 16 * k);
  }
  f32x16 acc;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = 0.f;
  // fragment set d holds k-step k + d; once used it is refilled with k-step
  // k + d + D (past the end: the last k-step again, in bounds, never used).
  // No branch inside the loop, so the compiler's waits stay per fragment.
  int k = 0;
  for (; k + D <= nk; k += D) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[d], fa[d], acc, 0, 0, 0);
      const int kn = min(k + d + D, nk - 1);
      fa[d] = *reinterpret_cast<const bf16x8 *>(ap + 16 * kn);
      fb[d] = *reinterpret_cast<const bf16x8 *>(wp + 16 * kn);
      __builtin_amdgcn_sched_barrier(0);  // keep each refill right after its MFMA
    }
  }
  // the last nk - k < D k-steps (a multiple of 4: K is a multiple of 64)
#pragma unroll
  for (int d = 0; d < D; d += 4) {
    if (k + d < nk) {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[d + e], fa[d + e], acc, 0, 0, 0);
    }
  }
  // lane holds row m0 + (lane & 31), register r column 8 (r / 4) + 4 (lane / 32) + r % 4
  const int64_t m = m0 + fr;
  if (m >= M) return;
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const int n = n0 + 8 * g + 4 * fh;
    if (n < N)
      epi_store4<EPI>(out, res, ldc, m, n, N, make_float4(acc[4 * g], acc[4 * g + 1], acc[4 * g + 2], acc[4 * g + 3]),
                      bias);
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

template <class C>
hipError_t go_bf16(const uint16_t *A, int lda, const uint16_t *W, const float *bias,
                   const float *res, void *out, int ldc, int M, int N, int K, int epi,
                   hipStream_t st) {
  if (K % C::BK) return hipErrorInvalidValue;
  const int tm = (M + C::BM - 1) / C::BM, tn = (N + C::BN - 1) / C::BN;
  const dim3 grid(tm * tn), block(C::NT);
  switch (epi) {
    case kEpiBias:
      gemm_bf16_kernel<C, kEpiBias><<<grid, block, 0, st>>>(A, lda, W, bias, res, out, ldc, M, N, K, tm, tn);
      break;
    case kEpiGelu:
      gemm_bf16_kernel<C, kEpiGelu><<<grid, block, 0, st>>>(A, lda, W, bias, res, out, ldc, M, N, K, tm, tn);
      break;
    case kEpiResidual:
      gemm_bf16_kernel<C, kEpiResidual><<<grid, block, 0, st>>>(A, lda, W, bias, res, out, ldc, M, N, K, tm, tn);
      break;
    case kEpiF32:
      gemm_bf16_kernel<C, kEpiF32><<<grid, block, 0, st>>>(A, lda, W, bias, res, out, ldc, M, N, K, tm, tn);
      break;
    case kEpiResidualFfn:
      gemm_bf16_kernel<C, kEpiResidualFfn><<<grid, block, 0, st>>>(A, lda, W, bias, res, out, ldc, M, N, K, tm, tn);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <class C, int PFD>
hipError_t go_pp(const uint16_t *A, int lda, const uint16_t *W, const float *bias,
                 const float *res, void *out, int ldc, int M, int N, int K, int epi,
                 hipStream_t st) {
  if (K % C::BK) return hipErrorInvalidValue;
  const int tm = (M + C::BM - 1) / C::BM, tn = (N + C::BN - 1) / C::BN;
  const dim3 grid(tm * tn), block(512);
  switch (epi) {
    case kEpiBias:
      gemm_pp_kernel<C, kEpiBias, PFD><<<grid, block, 0, st>>>(A, lda, W, bias, res, out, ldc, M, N, K, tm, tn);
      break;
    case kEpiGelu:
      gemm_pp_kernel<C, kEpiGelu, PFD><<<grid, block, 0, st>>>(A, lda, W, bias, res, out, ldc, M, N, K, tm, tn);
      break;
    case kEpiResidual:
      gemm_pp_kernel<C, kEpiResidual, PFD><<<grid, block, 0, st>>>(A, lda, W, bias, res, out, ldc, M, N, K, tm, tn);
      break;
    case kEpiF32:
      gemm_pp_kernel<C, kEpiF32, PFD><<<grid, block, 0, st>>>(A, lda, W, bias, res, out, ldc, M, N, K, tm, tn);
      break;
    case kEpiResidualFfn:
      gemm_pp_kernel<C, kEpiResidualFfn, PFD><<<grid, block, 0, st>>>(A, lda, W, bias, res, out, ldc, M, N, K, tm, tn);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <class C>
hipError_t go_sp(const uint16_t *A, int lda, const uint16_t *W, const float *bias,
                 const float *res, void *out, int ldc, int M, int N, int K, int epi,
                 hipStream_t st) {
  if (K % C::BK) return hipErrorInvalidValue;
  const int tm = (M + C::BM - 1) / C::BM, tn = (N + C::BN - 1) / C::BN;
  const dim3 grid(tm * tn), block(512);
  switch (epi) {
    case kEpiBias:
      gemm_sp_kernel<C, kEpiBias><<<grid, block, 0, st>>>(A, lda, W, bias, res, out, ldc, M, N, K, tm, tn);
      break;
    case kEpiGelu:
      gemm_sp_kernel<C, kEpiGelu><<<grid, block, 0, st>>>(A, lda, W, bias, res, out, ldc, M, N, K, tm, tn);
      break;
    case kEpiResidual:
      gemm_sp_kernel<C, kEpiResidual><<<grid, block, 0, st>>>(A, lda, W, bias, res, out, ldc, M, N, K, tm, tn);
      break;
    case kEpiF32:
      gemm_sp_kernel<C, kEpiF32><<<grid, block, 0, st>>>(A, lda, W, bias, res, out, ldc, M, N, K, tm, tn);
      break;
    case kEpiResidualFfn:
      gemm_sp_kernel<C, kEpiResidualFfn><<<grid, block, 0, st>>>(A, lda, W, bias, res, out, ldc, M, N, K, tm, tn);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

constexpr int kLatDepth = 16;  // k-steps of 16 in flight per wavefront (128 VGPRs of fragments)

hipError_t go_lat(const uint16_t *A, int lda, const uint16_t *W, const float *bias,
                  const float *res, void *out, int ldc, int M, int N, int K, int epi,
                  hipStream_t st) {
  if (K % 16) return hipErrorInvalidValue;
  const int tm = (M + 31) / 32, tn = (N + 31) / 32;
  const dim3 grid((unsigned)tm * tn), block(64);
  switch (epi) {
    case kEpiBias:
      gemm_lat_kernel<kEpiBias, kLatDepth><<<grid, block, 0, st>>>(A, lda, W, bias, res, out, ldc, M, N, K, tn);
      break;
    case kEpiGelu:
      gemm_lat_kernel<kEpiGelu, kLatDepth><<<grid, block, 0, st>>>(A, lda, W, bias, res, out, ldc, M, N, K, tn);
      break;
    case kEpiResidual:
      gemm_lat_kernel<kEpiResidual, kLatDepth><<<grid, block, 0, st>>>(A, lda, W, bias, res, out, ldc, M, N, K, tn);
      break;
    case kEpiF32:
      gemm_lat_kernel<kEpiF32, kLatDepth><<<grid, block, 0, st>>>(A, lda, W, bias, res, out, ldc, M, N, K, tn);
      break;
    case kEpiResidualFfn:
      gemm_lat_kernel<kEpiResidualFfn, kLatDepth><<<grid, block, 0, st>>>(A, lda, W, bias, res, out, ldc, M, N, K, tn);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// Tile configurations:
//   0  T1  128 x 64, register-staged, 4 waves (64 x 32 each), three blocks per CU
//   1  P1  128 x 128 ping-pong, 8 waves (64 x 32 each), two blocks per CU
//   2  P2  256 x 256 ping-pong, 8 waves (128 x 64 each), one block per CU
//   3  P3  128 x 384 ping-pong, 8 waves (64 x 96 each), one block per CU, A
//          prefetched to L2 one stage beyond the direct loads (P3 serves the
//          long-K, narrow-N products whose A rows stream from HBM; measured in
//          a layer sequence at 15880 x 768 x 3072: 125 -> 117 us.  For the
//          K = 768 products, whose A panels are shared by many column tiles
//          and already hit in L2, the same prefetch costs 5-10 %)
//   4  T0  32 x 64, register-staged, 2 waves (32 x 32 each): the pruned last
//          layer's GEMMs on one row per sequence (a few hundred rows), where
//          128 x 64 blocks would leave most CUs idle (380 x 768 x 3072:
//          27.2 -> 20.4 us)
//   5  S2  256 x 256 software-pipelined, 8 waves (128 x 64 each), one block
//          per CU, A triple-buffered (all 160 KiB of LDS) for N < 4096, double
//          buffered for wider products; it runs wherever the cost model below
//          picks a wide block (2 or 3)
//   6  L   32 x 32 per wavefront, one wavefront per block, operands straight
//          from memory into registers (latency tile for the smallest passes)
//                  BM  BN  BK WGM WGN PF MINW
using T1 = Cfg<128, 64, 64, 2, 2, 2, 3>;
using T0 = Cfg<32, 64, 64, 1, 2, 2, 3>;
using P1 = PPCfg<128, 128>;
using P2 = PPCfg<256, 256>;
using P3 = PPCfg<128, 384>;
using S2 = SPCfg<256, 256, 3>;
using S2w = SPCfg<256, 256, 2>;
static_assert(kGemmTiles == 7, "tile menu and launcher disagree");

constexpr int kCUs = 256;

}  // namespace

// Configuration for an M x N x K problem.  Blocks run in rounds of as many
// as are resident at once (128 x 128: two per CU; 256 x 256 and 128 x 384:
// one), and a round costs about as long as one block's work whatever the
// number of blocks in it, so the choice is mostly about how the last round
// is filled.  Cost of configuration c = rounds x (a_c + b_c K) microseconds,
// a partial last round counting (0.71 + 0.29 fill) of a full one, the GELU
// epilogue making a wide block's round 10 % longer; a_c, b_c fitted to a
// sweep of the model's shapes on MI355X (M = 2048 .. 16640 in steps of 256
// for K = 768 / 3072, 8192 .. 16384 in steps of 512 for K = 2048 / 8192;
// same-stream launches, time per launch):
//   shape (N x K, epilogue)     heuristic before -> this model, summed over M
//   2304 x 768 bias              2609 -> 2556 us
//   768 x 768 fp32               1185 -> 1157
//   3072 x 768 GELU              3937 -> 3982 (same tiles; run-to-run noise)
//   768 x 3072 fp32              3222 -> 3138
//   2048 x 2048 fp32             1877 -> 1825
//   2048 x 8192 fp32             6915 -> 6558
//   8192 x 2048 GELU             7307 -> 7274
//   6144 x 2048 bias             4707 -> 4801 (same tiles; noise)
// The 128 x 384 block is only considered for K >= 2048, and the wide blocks
// not at all when both N and K are below 2048.  Problems too small to give
// the 128 x 128 block half the CUs take the 128 x 64 block (more, smaller
// blocks), or the 32 x 64 block when even the 128 x 64 blocks would not
// cover the CUs.  Every configuration issues the
// same MFMA over K in the same order and K is never split, so each output's
// accumulation order does not depend on the configuration chosen or on the
// other sequences in the batch.
int gemm_tile_index(int M, int N, int K, int epi) {
  const int64_t b128 = (int64_t)((M + 127) / 128) * ((N + 127) / 128);
  // at most one 32 x 32 wavefront per CU: the latency tile (kernel time on
  // MI355X, TinyBERT at 64 rows: 4.7 -> 4.4 us QKV, 8.4 -> 6.9 us FFN2;
  // BERT-base FFN2 at 64 rows 16.6 -> 13.8 us; decoder FFN2 at one row 38.7
  // -> 30.6 us).  With more wavefronts than CUs its operand loads, 32 rows
  // of 32 bytes per instruction, queue in the CUs' address units and the
  // 32 x 64 block wins (decoder QKV at 256 rows: 18.7 vs 53.0 us).
  if (b128 < kCUs / 2 && (int64_t)((M + 31) / 32) * ((N + 31) / 32) <= kCUs) return 6;
  if (b128 < kCUs / 2) {
    const int64_t b128x64 = (int64_t)((M + 127) / 128) * ((N + 63) / 64);
    return b128x64 < kCUs ? 4 : 0;  // fewer 128 x 64 blocks than CUs: 32 x 64
  }
  // small N and K (the attention-out GEMM): the wide blocks time faster
  // alone but slower inside the layer sequence (15.9 k rows: 2.97 -> 3.1-3.25
  // ms per step), so the 128 x 128 block stays
  if (N < 2048 && K < 2048) return 1;
  struct Option { int tile, bm, bn, resident; double a, b; };
  static constexpr Option opts[] = {
      {1, 128, 128, 2 * kCUs, 4.5, 0.013},
      {2, 256, 256, kCUs, 11.69, 0.0205},
      {3, 128, 384, kCUs, 10.7, 0.0186},
  };
  const bool p3_fits = (N + 383) / 384 * 384 <= (N + 255) / 256 * 256;
  int best = 1;
  double best_cost = 0;
  for (const Option &o : opts) {
    if (o.tile == 3 && (!p3_fits || K < 2048)) continue;  // 128 x 384: long K only
    const int64_t blocks = (int64_t)((M + o.bm - 1) / o.bm) * ((N + o.bn - 1) / o.bn);
    const int64_t full = blocks / o.resident;
    const double fill = (double)(blocks - full * o.resident) / o.resident;
    const double rounds = (double)full + (fill > 0 ? 0.71 + 0.29 * fill : 0.0);
    double cost = rounds * (o.a + o.b * K);
    if (epi == kEpiGelu && o.tile != 1) cost *= 1.1;
    if (o.tile == 1 || cost < best_cost) {
      best = o.tile;
      best_cost = cost;
    }
  }
  // where a wide block wins, the software-pipelined 256 x 256 block does the
  // work: inside the layer sequence it matched or beat both wide ping-pong
  // blocks on every such shape (decoder at ~79 k rows per pass: attention-out
  // 115.0 -> 105.6 and FFN2 362.3 -> 339.4 ms per step, QKV and FFN1 equal;
  // BERT-base FFN2 6.34 -> 5.86 / 29.2 -> 26.3 ms per step on the short /
  // long-tail streams; same box)
  return best == 1 ? 1 : 5;
}

hipError_t launch_gemm_bf16_tile(int tile, const uint16_t *A, int lda, const uint16_t *W,
                                 const float *bias, const float *res, void *out, int ldc, int M,
                                 int N, int K, int epi, hipStream_t st) {
  if (M <= 0 || N <= 0) return hipSuccess;
  if (K <= 0 || K % 64) return hipErrorInvalidValue;
  switch (tile) {
    case 0: return go_bf16<T1>(A, lda, W, bias, res, out, ldc, M, N, K, epi, st);
    case 1: return go_pp<P1, 0>(A, lda, W, bias, res, out, ldc, M, N, K, epi, st);
    case 2: return go_pp<P2, 0>(A, lda, W, bias, res, out, ldc, M, N, K, epi, st);
    case 3:
      // W is padded to 256 rows; a 384-wide last column block must stay inside
      // that padding, else the 128 x 128 tile does the work (same result)
      if ((N + 383) / 384 * 384 > (N + 255) / 256 * 256)
        return go_pp<P1, 0>(A, lda, W, bias, res, out, ldc, M, N, K, epi, st);
      return go_pp<P3, 1>(A, lda, W, bias, res, out, ldc, M, N, K, epi, st);
    case 4: return go_bf16<T0>(A, lda, W, bias, res, out, ldc, M, N, K, epi, st);
    case 5:
      // two A buffers for the wide decoder products (N = 6144, 8192: QKV and
      // FFN1 inside the layer sequence 286 -> 277 and 415 -> 409 ms per step
      // on the decoder stream; QKV alone at 80 k rows 2.49e7 -> 2.28e7 busy
      // cycles); three for N <= 3072 (with two, the decoder's attention-out
      // and FFN2 took 104 -> 112 and 328 -> 348 ms per step and BERT-base's
      // QKV on the long-tail stream 24.5 -> 25.4 ms; BERT-base FFN2 at ~80 k
      // rows 857 -> 946 TFLOP/s with three)
      if (N >= 4096) return go_sp<S2w>(A, lda, W, bias, res, out, ldc, M, N, K, epi, st);
      return go_sp<S2>(A, lda, W, bias, res, out, ldc, M, N, K, epi, st);
    case 6: return go_lat(A, lda, W, bias, res, out, ldc, M, N, K, epi, st);
    default: return hipErrorInvalidValue;
  }
}

// The configuration from the cost model above (es_op_gemm_bf16_tile forces
// one, for tests and tuning sweeps).
hipError_t launch_gemm_bf16(const uint16_t *A, int lda, const uint16_t *W, const float *bias,
                            const float *res, void *out, int ldc, int M, int N, int K, int epi,
                            hipStream_t st) {
  return launch_gemm_bf16_tile(gemm_tile_index(M, N, K, epi), A, lda, W, bias, res, out, ldc, M, N,
                               K, epi, st);
}

hipError_t launch_gemm_split(const uint16_t *A, const uint16_t *W, const float *bias,
                             const float *res, float *out, uint16_t *outp, int ldc, int M, int N,
                             int K, int epi, hipStream_t st) {
  if (M <= 0 || N <= 0) return hipSuccess;
  if (K <= 0 || K % 64) return hipErrorInvalidValue;
  if (epi == kEpiGelu ? (N % 16 || !outp) : ((epi != kEpiF32 && epi != kEpiResidual) || !out || ldc < N))
    return hipErrorInvalidValue;
  // Up to 3 row tiles per block, as even as the row count allows, but at
  // least 192 blocks where fewer tiles per block give them (measured at 155
  // and 1024 rows of the decoder's shapes: 3 tiles best where the grid stays
  // large, 2 on the N = 2048 GEMMs at 155 rows, 4 never clearly better).
  const int mtiles = (M + 31) / 32, tn = (N + 31) / 32;
  int chunks = 1, mt = 1;
  for (int mx = 3; mx >= 1; --mx) {
    chunks = (mtiles + mx - 1) / mx;
    mt = (mtiles + chunks - 1) / chunks;
    if ((int64_t)chunks * tn >= 192) break;
  }
  // k-ranges of a multiple of 4 k-steps each
  const int kw = K % 256 == 0 ? 4 : K % 128 == 0 ? 2 : 1;
  const dim3 grid((unsigned)chunks * tn), block(64 * kw);
  auto go = [&](auto mtc) {
    constexpr int MT = decltype(mtc)::value, D = MT <= 2 ? 8 : 4;
    if (epi == kEpiF32)
      gemm_split_kernel<kEpiF32, MT, D><<<grid, block, 0, st>>>(A, W, bias, res, out, outp, ldc, M, N, K, tn);
    else if (epi == kEpiResidual)
      gemm_split_kernel<kEpiResidual, MT, D><<<grid, block, 0, st>>>(A, W, bias, res, out, outp, ldc, M, N, K, tn);
    else
      gemm_split_kernel<kEpiGelu, MT, D><<<grid, block, 0, st>>>(A, W, bias, res, out, outp, ldc, M, N, K, tn);
    return hipGetLastError();
  };
  switch (mt) {
    case 1: return go(std::integral_constant<int, 1>{});
    case 2: return go(std::integral_constant<int, 2>{});
    default: return go(std::integral_constant<int, 3>{});
  }
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
