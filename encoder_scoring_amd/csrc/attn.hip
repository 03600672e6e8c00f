// Masked attention over the packed, ragged batch, in two kernels around the
// Softmax row reduction (TurboTransformers review, Proposed method: Softmax
// is its own per-row "batch reduction" kernel):
//   scores:  S_ih[q, k] = (q_q . k_k) / sqrt(d)  for keys k of the same
//            sequence (all k < n_i, or k <= q when causal), fp32;
//   P = softmax(S) row by row (rowops.hip);
//   context: ctx[q, h*dp + e] = sum_k P_ih[q, k] v_k[h*dp + e].
// Work is a list of (sequence, 32-query-row tile) items built on the host,
// longest sequences first, times the heads on the second grid axis, so no
// block is spent on padding.  Score blocks follow score_row_off /
// score_block (kernels.h): n_i x ld_i per head, or the packed lower triangle
// when causal.
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
  const int64_t base = sbase[seq] + (int64_t)h * score_block(n, causal);
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
      if (q < n && k < n && (!causal || k <= q)) S[base + score_row_off(q, n, causal) + k] = acc[i] * scale;
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
  const int64_t base = sbase[seq] + (int64_t)h * score_block(n, causal);
  const Act *V = qkv + t0 * ldq + (2 * n_heads + h) * DP;
  const int e = tid % DP, r0 = tid / DP;
  float acc[NR] = {};
  const int kend = causal ? min(n, q0 + kQTile) : n;
  for (int k0 = 0; k0 < kend; k0 += 64) {
    __syncthreads();
    for (int x = tid; x < kQTile * 64; x += 256) {
      const int r = x >> 6, c = x & 63, q = q0 + r, k = k0 + c;
      const bool ok = q < n && k < n && (!causal || k <= q);
      sP[r][c] = ok ? to_f(P[base + score_row_off(q, n, causal) + k]) : 0.f;
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

// ---------------------------------------------------------------- bf16 MFMA
// One wavefront per (32-query tile, head).  Scores: S^T = K Q^T with
// v_mfma_f32_32x32x16_bf16, Q and K fragments read straight from the packed
// qkv rows (16 contiguous bytes per lane); with K as the first operand a lane
// ends up holding four consecutive keys of one query row, stored as one
// float4.  Context: ctx^T = V^T P^T; the V tile is transposed through LDS
// (keys contiguous per head dimension) and P rows are read directly.

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ bf16x8 ld_frag(const uint16_t *p) {
  return *reinterpret_cast<const bf16x8 *>(p);
}
__device__ __forceinline__ bf16x8 zero_frag() {
  bf16x8 z;
#pragma unroll
  for (int i = 0; i < 8; ++i) z[i] = (__bf16)0.0f;
  return z;
}

template <int DP>
__global__ __launch_bounds__(64) void scores_mfma_kernel(const uint16_t *__restrict__ qkv, int ldq,
                                                         int n_heads, float scale, int causal,
                                                         const int32_t *__restrict__ off,
                                                         const int64_t *__restrict__ sbase,
                                                         const int32_t *__restrict__ items,
                                                         float *__restrict__ S) {
  constexpr int KS = DP / 16;
  const int item = blockIdx.x, h = blockIdx.y, lane = threadIdx.x;
  const int seq = items[2 * item], q0 = items[2 * item + 1];
  const int64_t t0 = off[seq];
  const int n = off[seq + 1] - (int)t0;
  const int64_t base = sbase[seq] + (int64_t)h * score_block(n, causal);
  const int fr = lane & 31, fh = lane >> 5;
  const int q = q0 + fr;
  // rows are clamped to the sequence and the out-of-range fragments zeroed
  // after the load, so no load sits behind a branch and they overlap
  bf16x8 qf[KS];
  const uint16_t *Qr = qkv + (t0 + min(q, n - 1)) * ldq + h * DP + fh * 8;
#pragma unroll
  for (int kk = 0; kk < KS; ++kk) qf[kk] = ld_frag(Qr + kk * 16);
#pragma unroll
  for (int kk = 0; kk < KS; ++kk) qf[kk] = q < n ? qf[kk] : zero_frag();
  const int kend = causal ? min(n, q0 + kQTile) : n;
  float *Sr = S + base + score_row_off(q, n, causal);
  const int qlim = causal ? min(q + 1, n) : n;  // keys visible to this query row
  for (int k0 = 0; k0 < kend; k0 += 32) {
    const int k = k0 + fr;
    const uint16_t *Kr = qkv + (t0 + min(k, n - 1)) * ldq + (n_heads + h) * DP + fh * 8;
    bf16x8 kf[KS];
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) kf[kk] = ld_frag(Kr + kk * 16);
    f32x16 acc;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.f;
#pragma unroll
    for (int kk = 0; kk < KS; ++kk)
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k < n ? kf[kk] : zero_frag(), qf[kk], acc, 0, 0, 0);
    if (q >= n) continue;
    // lane holds keys k0 + 8 g + 4 fh + (0..3) of query q
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int kb = k0 + 8 * g + 4 * fh;
      const float4 v = make_float4(acc[4 * g] * scale, acc[4 * g + 1] * scale,
                                   acc[4 * g + 2] * scale, acc[4 * g + 3] * scale);
      if (kb + 3 < qlim) {
        *reinterpret_cast<float4 *>(Sr + kb) = v;
      } else {
        if (kb < qlim) Sr[kb] = v.x;
        if (kb + 1 < qlim) Sr[kb + 1] = v.y;
        if (kb + 2 < qlim) Sr[kb + 2] = v.z;
      }
    }
  }
}

// V tile of keys [k0, k0 + 32) of one head, staged into LDS transposed:
// sV[e * VP + key].  A lane loads 4 keys x 8 dims (four 16-byte reads along
// the key rows) and writes them as eight 8-byte rows of 4 keys, so the MFMA
// fragments below read keys contiguously.  Keys >= n become 0.  Loading and
// storing are separate steps so that a kernel can put the loads of a tile in
// flight together with its other loads before it waits.
// Lane u takes keys 4 (u % 8) .. + 3 and dims 8 (u / 8) .. + 7, so the 32
// lanes of one 8-byte LDS store cycle write 4 dim octets x 8 key quads.  The
// fused kernels use pitch kVPF = 36 (72 bytes): those stores then land on
// 16 oct + 18 d + 2 quad (mod 64) -- every bank once -- and the fragment
// reads of lanes r = 0..31 (8 bytes at row r) on 18 r (mod 64), also
// distinct.  With the earlier pitch of 40 and dim-octet-fastest lanes, a
// store hit each bank pair eight times (rocprofv3 on the decoder's
// attention: SQ_LDS_BANK_CONFLICT 1.56e8 cycles per launch, 37 % of the
// CUs' time).  The unfused P.V kernel reads 16-byte fragments and keeps the
// 16-byte aligned pitch kVP = 40.
constexpr int kVP = 40;   // pitch for 16-byte fragment reads (unfused P.V)
constexpr int kVPF = 36;  // pitch for the fused kernels' 8-byte reads (conflict-free)

template <int DP, int NTH = 64>
struct VtTile {
  static constexpr int OCT = DP / 8, UNITS = 8 * OCT, NU = (UNITS + NTH - 1) / NTH;
  uint4 r[NU][4];
};

// Keys at positions [0, np) come from rows Vp[0 .. np) (a shared prompt) and
// keys at positions >= np from Vs[key - np]; np = 0 for a plain sequence.
// Every lane reads a valid row (key clamped to n - 1, n >= 1) and store_vt
// zeroes keys >= n, so the loads need no branches.
template <int DP, int NTH = 64>
__device__ __forceinline__ void load_vt(VtTile<DP, NTH> &t, const uint16_t *__restrict__ Vp,
                                        const uint16_t *__restrict__ Vs, int np, int ldq, int k0,
                                        int n, int lane) {
  using T = VtTile<DP, NTH>;
#pragma unroll
  for (int i = 0; i < T::NU; ++i) {
    const int u = (lane + NTH * i) % T::UNITS, quad = u % 8, oct = u / 8;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int key = k0 + 4 * quad + j, kc = min(key, n - 1);
      const uint16_t *row = kc < np ? Vp + (int64_t)kc * ldq : Vs + (int64_t)(kc - np) * ldq;
      t.r[i][j] = *reinterpret_cast<const uint4 *>(row + oct * 8);
    }
  }
}

template <int DP, int VP, int NTH = 64>
__device__ __forceinline__ void store_vt(uint16_t *__restrict__ sV, VtTile<DP, NTH> &t, int k0, int n,
                                         int lane) {
  using T = VtTile<DP, NTH>;
#pragma unroll
  for (int i = 0; i < T::NU; ++i) {
    const int u = lane + NTH * i, quad = u % 8, oct = (u % T::UNITS) / 8;
    if (k0 + 32 > n) {  // only the last tile of a sequence has keys to clear
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (k0 + 4 * quad + j >= n) t.r[i][j] = make_uint4(0, 0, 0, 0);
    }
    if (T::UNITS % NTH == 0 || u < T::UNITS) {
#pragma unroll
      for (int d = 0; d < 8; ++d) {
        const int c = d >> 1, sh = (d & 1) * 16;
        auto pick = [&](const uint4 &x) {
          const uint32_t w = c == 0 ? x.x : c == 1 ? x.y : c == 2 ? x.z : x.w;
          return (w >> sh) & 0xffffu;
        };
        const uint2 w = make_uint2(pick(t.r[i][0]) | (pick(t.r[i][1]) << 16),
                                   pick(t.r[i][2]) | (pick(t.r[i][3]) << 16));
        *reinterpret_cast<uint2 *>(sV + (oct * 8 + d) * VP + 4 * quad) = w;
      }
    }
  }
}

// P.V: ctx^T = V^T P^T on MFMA.  P rows are read straight from global
// memory, 8 consecutive keys per lane; the V tile comes transposed from LDS.
template <int DP>
__global__ __launch_bounds__(64) void pv_mfma_kernel(const uint16_t *__restrict__ P,
                                                     const uint16_t *__restrict__ qkv, int ldq,
                                                     int n_heads, int causal,
                                                     const int32_t *__restrict__ off,
                                                     const int64_t *__restrict__ sbase,
                                                     const int32_t *__restrict__ items,
                                                     uint16_t *__restrict__ ctx, int ldc) {
  constexpr int NT = DP / 32;  // output column tiles
  __shared__ __attribute__((aligned(16))) uint16_t sV[DP * kVP];
  const int item = blockIdx.x, h = blockIdx.y, lane = threadIdx.x;
  const int seq = items[2 * item], q0 = items[2 * item + 1];
  const int64_t t0 = off[seq];
  const int n = off[seq + 1] - (int)t0;
  const int64_t base = sbase[seq] + (int64_t)h * score_block(n, causal);
  const int fr = lane & 31, fh = lane >> 5;
  const int q = q0 + fr;
  const int qlim = q < n ? (causal ? q + 1 : n) : 0;  // valid P entries of this row
  const uint16_t *Pr = P + base + score_row_off(q, n, causal);
  const uint16_t *V = qkv + t0 * ldq + (2 * n_heads + h) * DP;
  f32x16 acc[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[t][r] = 0.f;
  const int kend = causal ? min(n, q0 + kQTile) : n;
  for (int k0 = 0; k0 < kend; k0 += 32) {
    VtTile<DP> vt;
    load_vt<DP>(vt, V, V, 0, ldq, k0, n, lane);
    __syncthreads();
    store_vt<DP, kVP>(sV, vt, k0, n, lane);
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int kb = k0 + kk * 16 + fh * 8;  // first key of this lane's chunk
      bf16x8 pf;
      if (kb + 7 < qlim) {
        pf = ld_frag(Pr + kb);
      } else {
        pf = zero_frag();
        if (kb < qlim) {
          const bf16x8 raw = ld_frag(Pr + kb);
#pragma unroll
          for (int j = 0; j < 8; ++j)
            if (kb + j < qlim) pf[j] = raw[j];
        }
      }
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const bf16x8 vf = ld_frag(sV + (t * 32 + fr) * kVP + kk * 16 + fh * 8);
        acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf, acc[t], 0, 0, 0);
      }
    }
  }
  if (q >= n) return;
  uint16_t *Cr = ctx + (t0 + q) * ldc + h * DP;
  // lane holds head dims t*32 + 8 g + 4 fh + (0..3) of query q
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      uint2 u;
      u.x = f2bf2(acc[t][4 * g], acc[t][4 * g + 1]);
      u.y = f2bf2(acc[t][4 * g + 2], acc[t][4 * g + 3]);
      *reinterpret_cast<uint2 *>(Cr + t * 32 + 8 * g + 4 * fh) = u;
    }
}

// Fused attention for one (32-query tile, head): per 32-key tile, the scores
// S^T = K Q^T (MFMA), an online softmax (running max and sum per query,
// rescaling the context accumulator), and ctx^T += V^T P^T (MFMA) -- the
// score rows never leave registers.  With K as the first operand a lane
// holds keys k0 + 8 g + 4 fh + (0..3) of its query; the P.V MFMA is fed those
// registers directly by giving its 16 k-slots the key order
//   slots 0..3 -> keys 16 kk + 4 fh + (0..3),  slots 4..7 -> 16 kk + 8 + 4 fh + (0..3)
// and reading the transposed V tile in the same order (two 8-byte LDS reads).
// The contraction is order-free, so the result equals softmax(S) V up to
// rounding.
//
// The per-tile arithmetic of one wavefront's 32 queries lives in QueryTile,
// shared by the one-wavefront kernel (short sequences) and the four-wavefront
// kernel (long sequences, K and V staged once per block): a query's result
// does not depend on which kernel ran it.
template <int DP>
struct QueryTile {
  static constexpr int KS = DP / 16, NT = DP / 32;
  f32x16 acc[NT];
  float m_run, l_run;
  int q0, fr, fh;

  __device__ __forceinline__ void init(int q0_, int lane) {
    q0 = q0_;
    fr = lane & 31;
    fh = lane >> 5;
    m_run = -INFINITY;
    l_run = 0.f;
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[t][r] = 0.f;
  }
  // S^T tile of this wavefront's queries against 32 keys.
  __device__ __forceinline__ f32x16 scores(const bf16x8 (&kf)[KS], const bf16x8 (&qf)[KS]) const {
    f32x16 s;
#pragma unroll
    for (int r = 0; r < 16; ++r) s[r] = 0.f;
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[kk], qf[kk], s, 0, 0, 0);
    return s;
  }
  // Online-softmax update with key tile k0: s becomes the tile's
  // probabilities (unnormalised, relative to the reference m_run).
  // Masking only where a key of the tile can be invisible to a query of the
  // tile: the sequence's last key tile and, causal, tiles reaching past the
  // first query's position.  The first tile shows every query key 0, so
  // m_run is finite after it; a later tile whose keys are all masked for a
  // query leaves that query's reference, sum and accumulator exactly
  // unchanged (p = 0).  Scores are kept in base 2, s log2(e) / sqrt(d)
  // (sl2), so every probability is one v_exp_f32; the reference is kept in
  // scaled units (scaling by sl2 > 0 commutes with the max) and each
  // exponent is one fma: 2^(s sl2 - m).
  // The reference need not be the running max: the sum and the accumulator
  // are both relative to it, so the normalised result is the same for any
  // m_run.  It moves up to the tile's max only when that exceeds it by more
  // than kSlack (base-2 units, so every p stays <= 2^kSlack), and the
  // wavefront skips rescaling its accumulator (NT x 16 multiplies) when none
  // of its queries' references moved -- after the first key tiles, the
  // usual case.
  static constexpr float kSlack = 8.0f;
  __device__ __forceinline__ void update(f32x16 &s, int k0, int ntot, int np, bool causal, float sl2) {
    const int qpos = np + q0 + fr;
    if (k0 + 32 > ntot || (causal && k0 + 31 > np + q0)) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = k0 + 8 * (r >> 2) + 4 * fh + (r & 3);
        if (key >= ntot || (causal && key > qpos)) s[r] = -INFINITY;
      }
    }
    float mx = s[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[r]);
    mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));  // the other 16 keys of this query
    const float m_tile = mx * sl2;
    const bool move = m_tile > m_run + kSlack;  // always at the first tile (m_run = -inf)
    if (__any(move)) {
      const float m_new = move ? m_tile : m_run;
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);  // 1 where the reference stays
      l_run *= alpha;
      m_run = m_new;
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[t][r] *= alpha;
    }
    float psum = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      s[r] = __builtin_amdgcn_exp2f(fmaf(s[r], sl2, -m_run));
      psum += s[r];
    }
    l_run += psum;
  }
  // ctx^T += V^T P^T with the tile's V transposed in LDS (sV).
  __device__ __forceinline__ void pv(const f32x16 &p, const uint16_t *sV) {
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      bf16x8 pf;
#pragma unroll
      for (int j = 0; j < 8; ++j) pf[j] = (__bf16)p[8 * kk + j];
      const int c0 = 16 * kk + 4 * fh;  // tile keys of slots 0..3; slots 4..7 are c0 + 8
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const uint16_t *vr = sV + (t * 32 + fr) * kVPF + c0;
        const uint2 lo = *reinterpret_cast<const uint2 *>(vr);
        const uint2 hi = *reinterpret_cast<const uint2 *>(vr + 8);
        const bf16x8 vf = __builtin_bit_cast(bf16x8, make_uint4(lo.x, lo.y, hi.x, hi.y));
        acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf, acc[t], 0, 0, 0);
      }
    }
  }
  // Normalised context of the wavefront's valid queries (query < n).
  __device__ __forceinline__ void store(uint16_t *ctx, int ldc, int64_t t0, int n, int h) {
    const int q = q0 + fr;
    const float inv = 1.0f / (l_run + __shfl_xor(l_run, 32, kWave));
    if (q >= n) return;
    uint16_t *Cr = ctx + (t0 + q) * ldc + h * DP;
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        uint2 u;
        u.x = f2bf2(acc[t][4 * g] * inv, acc[t][4 * g + 1] * inv);
        u.y = f2bf2(acc[t][4 * g + 2] * inv, acc[t][4 * g + 3] * inv);
        *reinterpret_cast<uint2 *>(Cr + t * 32 + 8 * g + 4 * fh) = u;
      }
  }
};

// Key and query rows of a (sequence, head): with a shared prompt of np tokens
// at rows p0.., key position j < np is row p0 + j and position j >= np is the
// sequence's own row t0 + j - np; query q (own token q) sits at position
// np + q.  Key tiles stay aligned to position 0, so every query sees the same
// tiles, in the same order, as in the prompt + continuation laid out as one
// sequence.  Rows are clamped to the sequence, so no load sits behind a
// branch; values past the sequence are masked (K), zeroed (V) or never stored
// (queries).
struct HeadRows {
  const uint16_t *Qs, *Ks, *Kp, *Vs, *Vp;  // own rows (t0) and prompt rows (p0), this head
  int n, np, ntot;
  int64_t t0;
  int ldq;
  __device__ __forceinline__ const uint16_t *key_row(int k) const {  // k < ntot
    return k < np ? Kp + (int64_t)k * ldq : Ks + (int64_t)(k - np) * ldq;
  }
};

template <int DP, bool PFX>
__device__ __forceinline__ HeadRows head_rows(const uint16_t *qkv, int ldq, int n_heads, int h, int seq,
                                              const int32_t *off, const int32_t *pref,
                                              const int32_t *plen) {
  HeadRows r;
  r.t0 = off[seq];
  r.n = off[seq + 1] - (int)r.t0;
  r.np = PFX ? plen[seq] : 0;
  const int64_t p0 = PFX ? pref[seq] : 0;
  r.ntot = r.np + r.n;
  r.ldq = ldq;
  r.Qs = qkv + r.t0 * ldq + h * DP;
  r.Ks = qkv + r.t0 * ldq + (n_heads + h) * DP;
  r.Kp = qkv + p0 * ldq + (n_heads + h) * DP;
  r.Vs = qkv + r.t0 * ldq + (2 * n_heads + h) * DP;
  r.Vp = qkv + p0 * ldq + (2 * n_heads + h) * DP;
  return r;
}

template <int DP>
__device__ __forceinline__ void load_q(bf16x8 (&qf)[DP / 16], const HeadRows &hr, int q, int fh) {
  const uint16_t *Qr = hr.Qs + (int64_t)min(q, hr.n - 1) * hr.ldq + fh * 8;
#pragma unroll
  for (int kk = 0; kk < DP / 16; ++kk) qf[kk] = ld_frag(Qr + kk * 16);
#pragma unroll
  for (int kk = 0; kk < DP / 16; ++kk) qf[kk] = q < hr.n ? qf[kk] : zero_frag();
}

// One wavefront per (32-query tile, head): K fragments straight from the
// packed rows into registers, V transposed through LDS.
template <int DP, bool PFX>
__global__ __launch_bounds__(64) void attn_fused_kernel(const uint16_t *__restrict__ qkv, int ldq,
                                                        int n_heads, float scale, int causal,
                                                        const int32_t *__restrict__ off,
                                                        const int32_t *__restrict__ items,
                                                        const int32_t *__restrict__ pref,
                                                        const int32_t *__restrict__ plen,
                                                        uint16_t *__restrict__ ctx, int ldc) {
  constexpr int KS = DP / 16;
  __shared__ __attribute__((aligned(16))) uint16_t sV[DP * kVPF];
  const int item = blockIdx.x, h = blockIdx.y, lane = threadIdx.x;
  const int seq = items[2 * item], q0 = items[2 * item + 1];
  const HeadRows hr = head_rows<DP, PFX>(qkv, ldq, n_heads, h, seq, off, pref, plen);
  QueryTile<DP> qt;
  qt.init(q0, lane);
  bf16x8 qf[KS];
  load_q<DP>(qf, hr, q0 + qt.fr, qt.fh);
  const float sl2 = scale * 1.44269504088896340736f;
  const int kend = causal ? min(hr.ntot, hr.np + q0 + kQTile) : hr.ntot;
  // Each tile's K and V loads are in flight together; issuing the next
  // tile's loads ahead as well (a second register set) was measured slower:
  // the occupancy it costs outweighs the latency it hides.
  for (int k0 = 0; k0 < kend; k0 += 32) {
    bf16x8 kf[KS];
    const uint16_t *Kr = hr.key_row(min(k0 + qt.fr, hr.ntot - 1)) + qt.fh * 8;
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) kf[kk] = ld_frag(Kr + kk * 16);
    VtTile<DP> vt;
    load_vt<DP>(vt, hr.Vp, hr.Vs, hr.np, ldq, k0, hr.ntot, lane);
    __builtin_amdgcn_sched_barrier(0);  // every load of the tile issued before the first wait
    f32x16 s = qt.scores(kf, qf);
    __syncthreads();  // the previous tile's P.V reads of sV are done
    store_vt<DP, kVPF>(sV, vt, k0, hr.ntot, lane);
    qt.update(s, k0, hr.ntot, hr.np, causal != 0, sl2);
    __syncthreads();
    qt.pv(s, sV);
  }
  qt.store(ctx, ldc, hr.t0, hr.n, h);
}

// Four wavefronts per (128-query block, head) for long sequences: each key
// tile's K (swizzled rows) and V (transposed) go to LDS once and serve the
// four 32-query tiles, which otherwise each fetch them from L2.  Wavefront w
// owns queries [qb + 32 w, qb + 32 w + 32) and runs the same per-tile
// arithmetic (QueryTile) over the same key tiles as the one-wavefront
// kernel; wavefronts past the sequence or, causal, past their last visible
// key tile only help stage.
template <int DP, bool PFX>
__global__ __launch_bounds__(256) void attn_fused_mw_kernel(const uint16_t *__restrict__ qkv, int ldq,
                                                            int n_heads, float scale, int causal,
                                                            const int32_t *__restrict__ off,
                                                            const int32_t *__restrict__ items,
                                                            const int32_t *__restrict__ pref,
                                                            const int32_t *__restrict__ plen,
                                                            uint16_t *__restrict__ ctx, int ldc) {
  constexpr int KS = DP / 16, CPR = DP / 8, RPL = DP * 2 >= 256 ? 1 : 256 / (DP * 2);
  constexpr int KCH = 32 * CPR;                 // 16-byte chunks of a K tile
  constexpr int KPT = (KCH + 255) / 256;        // chunks per thread
  __shared__ __attribute__((aligned(16))) uint16_t sK[32 * DP];
  __shared__ __attribute__((aligned(16))) uint16_t sV[DP * kVPF];
  const int item = blockIdx.x, h = blockIdx.y, tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int seq = items[2 * item], qb = items[2 * item + 1];
  const HeadRows hr = head_rows<DP, PFX>(qkv, ldq, n_heads, h, seq, off, pref, plen);
  QueryTile<DP> qt;
  qt.init(qb + 32 * wave, lane);
  const bool active = qt.q0 < hr.n;
  bf16x8 qf[KS];
  load_q<DP>(qf, hr, qt.q0 + qt.fr, qt.fh);
  const float sl2 = scale * 1.44269504088896340736f;
  const int kend_blk = causal ? min(hr.ntot, hr.np + qb + 4 * kQTile) : hr.ntot;
  const int kend = causal ? min(hr.ntot, hr.np + qt.q0 + kQTile) : hr.ntot;
  // K chunk c of a tile: key c / CPR, 16-byte chunk c % CPR, stored at the
  // XOR-swizzled slot of its row (conflict-free fragment reads)
  auto swz = [](int row, int chunk) { return chunk ^ ((row / RPL) % CPR); };
  // Every thread stages part of each key tile: KPT 16-byte K chunks and, for
  // the first VT threads, one 4-key x 8-dim unit of V.  The next tile's
  // loads are issued right after the current tile is written to LDS, so they
  // are in flight while the current tile is computed.
  using VT = VtTile<DP, 256>;
  constexpr int VTH = (VT::UNITS + 63) / 64 * 64;  // whole wavefronts that load V
  uint4 kr[KPT];
  VT vt;
  auto load_tile = [&](int k0) {
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int c = (tid + 256 * i) % KCH, key = c / CPR, ch = c % CPR;
      kr[i] = *reinterpret_cast<const uint4 *>(hr.key_row(min(k0 + key, hr.ntot - 1)) + ch * 8);
    }
    if (tid < VTH) load_vt<DP, 256>(vt, hr.Vp, hr.Vs, hr.np, ldq, k0, hr.ntot, tid);
  };
  load_tile(0);
  for (int k0 = 0; k0 < kend_blk; k0 += 32) {
    __syncthreads();  // the previous tile's reads of sK and sV are done
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int c = tid + 256 * i, key = (c % KCH) / CPR, ch = c % CPR;
      if (KCH % 256 == 0 || c < KCH)
        *reinterpret_cast<uint4 *>(sK + key * DP + (swz(key, ch) << 3)) = kr[i];
    }
    if (tid < VTH) store_vt<DP, kVPF, 256>(sV, vt, k0, hr.ntot, tid);
    if (k0 + 32 < kend_blk) load_tile(k0 + 32);
    __syncthreads();
    if (active && k0 < kend) {
      bf16x8 kf[KS];
#pragma unroll
      for (int kk = 0; kk < KS; ++kk)
        kf[kk] = *reinterpret_cast<const bf16x8 *>(sK + qt.fr * DP + (swz(qt.fr, kk * 2 + qt.fh) << 3));
      f32x16 s = qt.scores(kf, qf);
      qt.update(s, k0, hr.ntot, hr.np, causal != 0, sl2);
      qt.pv(s, sV);
    }
  }
  if (active) qt.store(ctx, ldc, hr.t0, hr.n, h);
}

// Shared-prompt candidates, four 32-query tiles of candidates of the same
// prompt per block (wavefront w: items[8 b + 2 w], sequence < 0 = empty).
// Key tiles that lie wholly inside the prompt (k0 + 32 <= np) are the same for
// all four and are staged in LDS once, as in the four-wavefront kernel; the
// remaining tiles (the one holding the prompt's end and the candidate's own
// keys) differ per wavefront, which then works alone as the one-wavefront
// kernel does, with its own V region and no block barrier.  Per query, the
// same key tiles in the same order and the same per-tile arithmetic
// (QueryTile) as the other two kernels.
template <int DP>
__global__ __launch_bounds__(256) void attn_fused_pfx_kernel(const uint16_t *__restrict__ qkv, int ldq,
                                                             int n_heads, float scale, int causal,
                                                             const int32_t *__restrict__ off,
                                                             const int32_t *__restrict__ items,
                                                             const int32_t *__restrict__ pref,
                                                             const int32_t *__restrict__ plen,
                                                             uint16_t *__restrict__ ctx, int ldc) {
  constexpr int KS = DP / 16, CPR = DP / 8, RPL = DP * 2 >= 256 ? 1 : 256 / (DP * 2);
  constexpr int KCH = 32 * CPR, KPT = (KCH + 255) / 256;
  __shared__ __attribute__((aligned(16))) uint16_t sK[32 * DP];
  __shared__ __attribute__((aligned(16))) uint16_t sV[DP * kVPF];
  __shared__ __attribute__((aligned(16))) uint16_t sVw[4][DP * kVPF];
  const int item = blockIdx.x, h = blockIdx.y, tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int seq = items[8 * item + 2 * wave], q0 = items[8 * item + 2 * wave + 1];
  const bool active = seq >= 0;
  // the block's prompt (every non-empty slot shares it; slot 0 is never empty)
  const int seq0 = items[8 * item];
  const int np = plen[seq0];
  const HeadRows hr = head_rows<DP, true>(qkv, ldq, n_heads, h, active ? seq : seq0, off, pref, plen);
  QueryTile<DP> qt;
  qt.init(q0, lane);
  bf16x8 qf[KS];
  load_q<DP>(qf, hr, q0 + qt.fr, qt.fh);
  const float sl2 = scale * 1.44269504088896340736f;
  auto swz = [](int row, int chunk) { return chunk ^ ((row / RPL) % CPR); };
  // prompt tiles, shared: keys [0, kp), staged by every thread with the next
  // tile's loads in flight, as in the four-wavefront kernel
  const int kp = np / 32 * 32;
  using VT = VtTile<DP, 256>;
  constexpr int VTH = (VT::UNITS + 63) / 64 * 64;
  uint4 kr[KPT];
  VT vt;
  auto load_tile = [&](int k0) {
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int c = (tid + 256 * i) % KCH, key = c / CPR, ch = c % CPR;
      kr[i] = *reinterpret_cast<const uint4 *>(hr.key_row(k0 + key) + ch * 8);
    }
    if (tid < VTH) load_vt<DP, 256>(vt, hr.Vp, hr.Vs, hr.np, ldq, k0, hr.ntot, tid);
  };
  if (kp > 0) load_tile(0);
  for (int k0 = 0; k0 < kp; k0 += 32) {
    __syncthreads();  // the previous tile's reads of sK and sV are done
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int c = tid + 256 * i, key = (c % KCH) / CPR, ch = c % CPR;
      if (KCH % 256 == 0 || c < KCH)
        *reinterpret_cast<uint4 *>(sK + key * DP + (swz(key, ch) << 3)) = kr[i];
    }
    if (tid < VTH) store_vt<DP, kVPF, 256>(sV, vt, k0, hr.ntot, tid);
    if (k0 + 32 < kp) load_tile(k0 + 32);
    __syncthreads();
    if (active) {
      bf16x8 kf[KS];
#pragma unroll
      for (int kk = 0; kk < KS; ++kk)
        kf[kk] = *reinterpret_cast<const bf16x8 *>(sK + qt.fr * DP + (swz(qt.fr, kk * 2 + qt.fh) << 3));
      f32x16 s = qt.scores(kf, qf);
      qt.update(s, k0, hr.ntot, hr.np, causal != 0, sl2);
      qt.pv(s, sV);
    }
  }
  if (!active) return;  // no block barrier follows
  // the wavefront's own tiles: keys [kp, kend)
  const int kend = causal ? min(hr.ntot, hr.np + q0 + kQTile) : hr.ntot;
  uint16_t *myV = sVw[wave];
  for (int k0 = kp; k0 < kend; k0 += 32) {
    bf16x8 kf[KS];
    const uint16_t *Kr = hr.key_row(min(k0 + qt.fr, hr.ntot - 1)) + qt.fh * 8;
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) kf[kk] = ld_frag(Kr + kk * 16);
    VtTile<DP> vt;
    load_vt<DP>(vt, hr.Vp, hr.Vs, hr.np, ldq, k0, hr.ntot, lane);
    __builtin_amdgcn_sched_barrier(0);
    f32x16 s = qt.scores(kf, qf);
    // myV belongs to this wavefront alone, so fences (no barrier) order the
    // previous tile's reads of it before these writes and these writes
    // before this tile's reads (lanes exchange keys through it)
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    store_vt<DP, kVPF>(myV, vt, k0, hr.ntot, lane);
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "workgroup");
    qt.update(s, k0, hr.ntot, hr.np, causal != 0, sl2);
    qt.pv(s, myV);
  }
  qt.store(ctx, ldc, hr.t0, hr.n, h);
}

// Last-token attention in fp32, for the refinement of the reward rows: the
// query, and the key and value of the last token itself, come from the fp32
// row of that token (ql: row i = sequence i, Q | K | V at the bulk layout's
// columns, pitch ldl); every other key / value is the bulk layer's bf16 row
// (shared prompt rows first, as in the fused kernels).  The last query sees
// every key of its sequence under either mask.  One block of four wavefronts
// per (sequence, head), a head's sequences in order on one XCD (the
// candidates of a shared prompt then read its keys and values from one L2).
// A key's DP dims are split over DP / 8 neighbouring lanes, 16 bytes each,
// so a wavefront instruction reads whole rows (one 256-byte row per 16 lanes
// at DP = 128) and the block takes 256 / (DP / 8) keys at once; a key's dot
// product is 8 fmas per lane and a butterfly over its lanes.  Max and sum reduce over the block; P . V runs on the same
// lane split, each key slot accumulating its keys in ascending order, and
// the slots are summed in fixed order through LDS, so the result is
// reproducible.  Writes columns [h dp, h dp + dp) of row i of ctx in the
// split-operand layout (split_off, K = kc), the input of the output
// projection's split GEMM; the head of index 0 also zeroes columns
// [n_heads dp, kc), the band a wider GEMM K reads.
constexpr int kLastMaxKeys = kLastMaxKeysHost;
constexpr int kLastThreads = 256;

template <int DP>
__global__ __launch_bounds__(kLastThreads) void attn_last_kernel(
    const uint16_t *__restrict__ qkv, int ldq, const float *__restrict__ ql, int ldl, int n_heads,
    float scale, const int32_t *__restrict__ off, const int32_t *__restrict__ pref,
    const int32_t *__restrict__ plen, uint16_t *__restrict__ ctx, int kc) {
  constexpr int CH = DP / 8, G = kLastThreads / CH, NW = kLastThreads / kWave;
  static_assert(CH <= kWave && kWave % CH == 0, "a key's lanes lie in one wavefront");
  __shared__ float sp[kLastMaxKeys];
  __shared__ __align__(16) float red[G * DP];
  __shared__ float wred[2 * NW];
  // sequences of one head run together on one XCD: a shared prompt's keys
  // and values then come from that XCD's L2 for all its candidates
  const int item = xcd_contiguous(blockIdx.x, gridDim.x);
  // sequences in packed order: the bulk attention, which runs just before
  // and walks the longest first, read the first (shortest, the plan being
  // sorted) last, so their keys and values are the likeliest still in the MALL
  const int n_seqs = gridDim.x / n_heads, seq = item % n_seqs, h = item / n_seqs;
  const int t = threadIdx.x;
  const int c = t % CH, g = t / CH, lane = t % kWave, wv = t / kWave;
  const int t0 = off[seq], n = off[seq + 1] - off[seq];
  const int np = plen ? plen[seq] : 0, p0 = pref ? pref[seq] : 0;
  const int L = np + n;  // keys of the last query, its own last
  const int kq = h * DP + 8 * c, kk = n_heads * DP + h * DP + 8 * c, kv = 2 * n_heads * DP + h * DP + 8 * c;
  const float *qrow = ql + (int64_t)seq * ldl;
  float q[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) q[e] = qrow[kq + e];
  auto row = [&](int j) { return qkv + (int64_t)(j < np ? p0 + j : t0 + j - np) * ldq; };
  auto unpack = [](const uint4 &u, float (&v)[8]) {
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[2 * e] = bf2f(w[e] & 0xffffu);
      v[2 * e + 1] = bf2f(w[e] >> 16);
    }
  };
  // Keys in batches of U per key slot, all U loads issued before any use:
  // the rows are read at min(j, L - 1) (always a row of the sequence) and
  // position L - 1 takes the fp32 key instead.
  constexpr int U = 8;
  float mx = -INFINITY;
  for (int j0 = g; j0 < L; j0 += U * G) {
    uint4 kb[U];
#pragma unroll
    for (int u = 0; u < U; ++u) kb[u] = *reinterpret_cast<const uint4 *>(row(min(j0 + u * G, L - 1)) + kk);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = j0 + u * G;
      if (j >= L) break;  // the same for a key's CH lanes
      float k[8];
      if (j == L - 1) {
#pragma unroll
        for (int e = 0; e < 8; ++e) k[e] = qrow[kk + e];
      } else {
        unpack(kb[u], k);
      }
      float dot = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) dot = fmaf(q[e], k[e], dot);
#pragma unroll
      for (int o = CH / 2; o > 0; o >>= 1) dot += __shfl_xor(dot, o, kWave);
      const float sc = dot * scale;
      if (c == 0) sp[j] = sc;
      mx = fmaxf(mx, sc);
    }
  }
  mx = wave_max(mx);
  if (lane == 0) wred[wv] = mx;
  __syncthreads();  // scores and per-wavefront maxima in LDS
  mx = wred[0];
#pragma unroll
  for (int w = 1; w < NW; ++w) mx = fmaxf(mx, wred[w]);
  float sum = 0.f;
  for (int j = t; j < L; j += kLastThreads) {
    const float pj = expf(sp[j] - mx);
    sp[j] = pj;
    sum += pj;
  }
  sum = wave_sum(sum);
  if (lane == 0) wred[NW + wv] = sum;
  __syncthreads();  // probabilities and per-wavefront sums in LDS
  sum = wred[NW];
#pragma unroll
  for (int w = 1; w < NW; ++w) sum += wred[NW + w];
  float acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.f;
  for (int j0 = g; j0 < L; j0 += U * G) {
    uint4 vb[U];
#pragma unroll
    for (int u = 0; u < U; ++u) vb[u] = *reinterpret_cast<const uint4 *>(row(min(j0 + u * G, L - 1)) + kv);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = j0 + u * G;
      if (j >= L) break;
      float v[8];
      if (j == L - 1) {
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = qrow[kv + e];
      } else {
        unpack(vb[u], v);
      }
      const float pj = sp[j];
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] = fmaf(pj, v[e], acc[e]);
    }
  }
  // red[g][8 c + e]: thread t's 8 values at 8 t
  *reinterpret_cast<float4 *>(red + 8 * t) = make_float4(acc[0], acc[1], acc[2], acc[3]);
  *reinterpret_cast<float4 *>(red + 8 * t + 4) = make_float4(acc[4], acc[5], acc[6], acc[7]);
  __syncthreads();
  const float inv = 1.0f / sum;
  for (int o = t; o < DP / 4; o += kLastThreads) {  // 4 dims per thread, slots in order
    float v[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float a = red[4 * o + e];
      for (int s2 = 1; s2 < G; ++s2) a += red[s2 * DP + 4 * o + e];
      v[e] = a * inv;
    }
    uint2 hi, lo;
    split4(v, hi, lo);
    *reinterpret_cast<uint2 *>(ctx + split_off(seq, h * DP + 4 * o, kc, 0)) = hi;
    *reinterpret_cast<uint2 *>(ctx + split_off(seq, h * DP + 4 * o, kc, 1)) = lo;
  }
  if (h == 0)
    for (int c4 = n_heads * DP / 4 + t; c4 < kc / 4; c4 += kLastThreads) {
      *reinterpret_cast<uint2 *>(ctx + split_off(seq, 4 * c4, kc, 0)) = make_uint2(0, 0);
      *reinterpret_cast<uint2 *>(ctx + split_off(seq, 4 * c4, kc, 1)) = make_uint2(0, 0);
    }
}

template <typename F>
hipError_t dispatch_dp(int dp, F &&f) {
  switch (dp) {
    case 32: return f(std::integral_constant<int, 32>{});
    case 64: return f(std::integral_constant<int, 64>{});
    case 128: return f(std::integral_constant<int, 128>{});
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_scores(bool act_bf16, const void *qkv, int ldq, int n_heads, int dp, float scale,
                         bool causal, const Ragged &r, float *S, hipStream_t st) {
  if (r.plen) return hipErrorInvalidValue;  // shared prompts: fused attention only
  if (r.n_items <= 0) return hipSuccess;
  const dim3 grid(r.n_items, n_heads), block(256);
  return dispatch_dp(dp, [&](auto dpc) {
    constexpr int DP = decltype(dpc)::value;
    if (act_bf16)
      scores_mfma_kernel<DP><<<grid, dim3(64), 0, st>>>((const uint16_t *)qkv, ldq, n_heads, scale,
                                                        causal ? 1 : 0, r.off, r.sbase, r.items, S);
    else
      scores_kernel<float, DP><<<grid, block, 0, st>>>((const float *)qkv, ldq, n_heads, scale,
                                                       causal ? 1 : 0, r.off, r.sbase, r.items, S);
    return hipGetLastError();
  });
}

hipError_t launch_pv(bool act_bf16, const void *P, const void *qkv, int ldq, int n_heads, int dp,
                     bool causal, const Ragged &r, void *ctx, int ldc, hipStream_t st) {
  if (r.plen) return hipErrorInvalidValue;  // shared prompts: fused attention only
  if (r.n_items <= 0) return hipSuccess;
  const dim3 grid(r.n_items, n_heads), block(256);
  return dispatch_dp(dp, [&](auto dpc) {
    constexpr int DP = decltype(dpc)::value;
    if (act_bf16)
      pv_mfma_kernel<DP><<<grid, dim3(64), 0, st>>>((const uint16_t *)P, (const uint16_t *)qkv, ldq,
                                                    n_heads, causal ? 1 : 0, r.off, r.sbase,
                                                    r.items, (uint16_t *)ctx, ldc);
    else
      pv_kernel<float, float, DP><<<grid, block, 0, st>>>((const float *)P, (const float *)qkv, ldq,
                                                          n_heads, causal ? 1 : 0, r.off, r.sbase,
                                                          r.items, (float *)ctx, ldc);
    return hipGetLastError();
  });
}

hipError_t launch_attn_fused(const uint16_t *qkv, int ldq, int n_heads, int dp, float scale,
                             bool causal, const Ragged &r, uint16_t *ctx, int ldc, hipStream_t st) {
  if ((r.plen != nullptr) != (r.pref != nullptr)) return hipErrorInvalidValue;
  // long sequences on the four-wavefront kernel, the rest one wavefront per tile
  const int32_t *sw = r.fused_items ? r.fused_items : r.items;
  const int n_sw = r.fused_items ? r.n_fused_items : r.n_items;
  const int n_mw = r.fused_items ? r.n_mw_items : 0;
  return dispatch_dp(dp, [&](auto dpc) {
    constexpr int DP = decltype(dpc)::value;
    const int c = causal ? 1 : 0;
    if (n_sw > 0) {
      const dim3 grid(n_sw, n_heads);
      if (r.plen)
        attn_fused_kernel<DP, true><<<grid, dim3(64), 0, st>>>(qkv, ldq, n_heads, scale, c, r.off, sw,
                                                               r.pref, r.plen, ctx, ldc);
      else
        attn_fused_kernel<DP, false><<<grid, dim3(64), 0, st>>>(qkv, ldq, n_heads, scale, c, r.off, sw,
                                                                nullptr, nullptr, ctx, ldc);
    }
    if (r.plen && r.n_pfx_items > 0) {
      const dim3 grid(r.n_pfx_items, n_heads);
      attn_fused_pfx_kernel<DP><<<grid, dim3(256), 0, st>>>(qkv, ldq, n_heads, scale, c, r.off,
                                                             r.pfx_items, r.pref, r.plen, ctx, ldc);
    }
    if (n_mw > 0) {
      const dim3 grid(n_mw, n_heads);
      if (r.plen)
        attn_fused_mw_kernel<DP, true><<<grid, dim3(256), 0, st>>>(qkv, ldq, n_heads, scale, c, r.off,
                                                                   r.mw_items, r.pref, r.plen, ctx, ldc);
      else
        attn_fused_mw_kernel<DP, false><<<grid, dim3(256), 0, st>>>(qkv, ldq, n_heads, scale, c, r.off,
                                                                    r.mw_items, nullptr, nullptr, ctx, ldc);
    }
    return hipGetLastError();
  });
}

hipError_t launch_attn_last(const uint16_t *qkv, int ldq, const float *ql, int ldl, int n_heads,
                            int dp, float scale, const Ragged &r, uint16_t *ctx, int kc,
                            hipStream_t st) {
  if (r.n_seqs <= 0) return hipSuccess;
  if ((int64_t)r.n_seqs * n_heads > INT32_MAX || r.max_len > kLastMaxKeys) return hipErrorInvalidValue;
  if ((r.plen != nullptr) != (r.pref != nullptr) || r.max_len <= 0 || kc < n_heads * dp || kc % 16 ||
      ldl < 3 * n_heads * dp)
    return hipErrorInvalidValue;
  return dispatch_dp(dp, [&](auto dpc) {
    constexpr int DP = decltype(dpc)::value;
    attn_last_kernel<DP><<<dim3(r.n_seqs * n_heads), dim3(kLastThreads), 0, st>>>(qkv, ldq, ql, ldl, n_heads, scale,
                                                                      r.off, r.pref, r.plen, ctx, kc);
    return hipGetLastError();
  });
}

}  // namespace es
