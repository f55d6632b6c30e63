// Device pieces shared by the decode-attention kernels (attend.hip,
// attend_rc.hip): the query-side smoothing of the dual transform and the
// dense fp16 window partial.
#pragma once
#include "kvq_internal.h"

namespace kvq {

// Dual transform: the keys were coded divided channel-wise by the factor row
// of their (sequence, KV head); multiplying the query's channels by the same
// row before the rotation leaves every score unchanged.  v: the 8 channels
// at col*8 of one query row.
template <int D>
__device__ __forceinline__ void smooth_query(float (&v)[8], const float* __restrict__ ksm, int b,
                                             int kv, int Hkv, int64_t rows, int col) {
  const float4* lp = reinterpret_cast<const float4*>(
      ksm + (((int64_t)b * Hkv + kv) % rows) * D + col * 8);
  const float4 a = lp[0], c = lp[1];
  v[0] *= a.x; v[1] *= a.y; v[2] *= a.z; v[3] *= a.w;
  v[4] *= c.x; v[5] *= c.y; v[6] *= c.z; v[7] *= c.w;
}

// Window block: softmax partial (m, l, o) of up to WB (ATTN_WIN_BLOCK) fp16 window
// tokens [w0, w1) for the RP query heads of a unit, o rotated like the coded
// tokens' (H v / sqrt(D)) so the merge treats every record alike.
// L = D/8 lanes per token row (8 dims per lane, 16-byte loads); pass A
// stores the scores in LDS, pass B accumulates p * v per row, rows are summed
// within each wave by lane exchanges and across waves through LDS.
template <int RP, int D, int WB = ATTN_WIN_BLOCK>
__device__ __forceinline__ void window_partial(const float* __restrict__ q,
                                               const uint16_t* __restrict__ kw,
                                               const uint16_t* __restrict__ vw,
                                               float* __restrict__ part, uint8_t* smem, int b,
                                               int kv, int h0, int nh, int Hq, int Hkv,
                                               int wstride, int w0, int w1, int slot, int nslots,
                                               int pstride, float scale) {
  constexpr int L = D / 8;
  constexpr int ROWS = 512 / L;
  float* ssc = reinterpret_cast<float*>(smem);                  // [WB][RP]
  float* wacc = ssc + WB * RP;                                  // [8 waves][RP][D]
  __shared__ float wred[8][RP];
  __shared__ float wm[RP];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int row = tid / L, col = tid % L;
  const uint16_t* kwp = kw + ((int64_t)b * Hkv + kv) * wstride * D + col * 8;
  const uint16_t* vwp = vw + ((int64_t)b * Hkv + kv) * wstride * D + col * 8;
  float qv[RP][8];
#pragma unroll
  for (int r = 0; r < RP; ++r) {
    const float* qp = q + ((int64_t)b * Hq + h0 + (r < nh ? r : nh - 1)) * D + col * 8;
#pragma unroll
    for (int e = 0; e < 8; ++e) qv[r][e] = qp[e] * scale;
  }
  const int n = w1 - w0;
  // A block of at most one row pass (WB <= ROWS) loads its V row with its K
  // row, so q, K and V come back in one round trip.
  constexpr bool ONE = WB <= ROWS;
  float vx1[8];
  // pass A: scores (the row sums' lane exchanges keep this loop rolled)
  for (int i = 0; i < n; i += ROWS) {                 // uniform trip count
    const int w = i + row;
    const int wl = w < n ? w : n - 1;
    float kx[8];
    load8<2>(kwp + (int64_t)(w0 + wl) * D, kx);
    if constexpr (ONE) load8<2>(vwp + (int64_t)(w0 + wl) * D, vx1);
#pragma unroll
    for (int r = 0; r < RP; ++r) {
      float dot = 0.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e) dot = __builtin_fmaf(qv[r][e], kx[e], dot);
      dot = row_sum<L>(dot);
      if (w < n && col == 0) ssc[w * RP + r] = dot;
    }
  }
  __syncthreads();
  float m[RP];
#pragma unroll
  for (int r = 0; r < RP; ++r) {
    float v = -__builtin_inff();
    for (int t = tid; t < n; t += 512) v = fmaxf(v, ssc[t * RP + r]);
    v = wave_max(v);
    if (lane == 0) wred[wave][r] = v;
  }
  __syncthreads();
  if (tid < RP) {
    float v = wred[0][tid];
    for (int w = 1; w < 8; ++w) v = fmaxf(v, wred[w][tid]);
    wm[tid] = v;
  }
  __syncthreads();
#pragma unroll
  for (int r = 0; r < RP; ++r) m[r] = wm[r];
  // pass B: weights and p * v
  float acc[RP][8], ls[RP];
#pragma unroll
  for (int r = 0; r < RP; ++r) {
    ls[r] = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[r][e] = 0.0f;
  }
#pragma unroll 4
  for (int i = 0; i < n; i += ROWS) {
    const int w = i + row;
    if (w < n) {
      float vx[8];
      if constexpr (ONE) {
#pragma unroll
        for (int e = 0; e < 8; ++e) vx[e] = vx1[e];
      } else {
        load8<2>(vwp + (int64_t)(w0 + w) * D, vx);
      }
#pragma unroll
      for (int r = 0; r < RP; ++r) {
        const float pw = __expf(ssc[w * RP + r] - m[r]);
        ls[r] += pw;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[r][e] = __builtin_fmaf(pw, vx[e], acc[r][e]);
      }
    }
  }
  // into the coded (rotated) domain, H sum p v = sum p H v: the L lanes of a
  // row group hold sums over the same rows
  constexpr float rs = rsqrt_pow2(D);
#pragma unroll
  for (int r = 0; r < RP; ++r) {
    hadamard_row<8, L>(acc[r], lane);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[r][e] *= rs;
  }
  // rows of a wave -> one row (lanes L apart), then waves through LDS
#pragma unroll
  for (int r = 0; r < RP; ++r) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {                     // lanes of one column: L .. 32 apart
      if constexpr (L <= 8) acc[r][e] += xor_lane<8>(acc[r][e]);
      if constexpr (L <= 16) acc[r][e] = pair_sum<16>(acc[r][e]);
      acc[r][e] = pair_sum<32>(acc[r][e]);
    }
    ls[r] = wave_sum(col == 0 ? ls[r] : 0.0f);
  }
  if (lane < L) {
#pragma unroll
    for (int r = 0; r < RP; ++r)
#pragma unroll
      for (int e = 0; e < 8; ++e) wacc[(wave * RP + r) * D + col * 8 + e] = acc[r][e];
  }
  if (lane == 0) {
#pragma unroll
    for (int r = 0; r < RP; ++r) wred[wave][r] = ls[r];
  }
  __syncthreads();
  for (int o = tid; o < RP * D; o += 512) {
    const int r = o / D, d = o - r * D;
    if (r >= nh) continue;
    float v = 0.0f;
    for (int w = 0; w < 8; ++w) v += wacc[(w * RP + r) * D + d];
    float* pp = part + ((int64_t)(b * Hq + h0 + r) * nslots + slot) * pstride;
    pp[4 + d] = v;
    if (d == 0) {
      float l = 0.0f;
      for (int w = 0; w < 8; ++w) l += wred[w][r];
      pp[0] = m[r];
      pp[1] = l;
    }
  }
}

}  // namespace kvq
