// K4/K5 -- single-token decode attention over uint8 codes plus an fp16
// recency window.
//
//   * The query is rotated once, q_rot = H_D q: the inverse rotation of the
//     keys is absorbed into the query ("VeloxQuant-MLX 0.5.1", VecInfer).
//   * Keys are scored in the compressed domain through a per-query table
//     LUT[s][g][c] = scale * q_rot_g . C^K_sg[c], so K is never materialised
//     ("Differential-KV" README, Decode & Prefill Innovations, query scoring
//     in the compressed subspace).
//   * Values are accumulated in the rotated domain as a per-(s, g) histogram
//     of softmax weights, W_sg[c] = sum_t p_t [z_tsg == c], and contracted
//     once per chunk: o_rot = sum_sg sum_c W_sg[c] C^V_sg[c].
//   * The token axis is split into chunks (split-K); each chunk emits an
//     fp32 partial (m, l, o_rot) and the merge kernel combines the chunks and
//     the dense fp16 window by log-sum-exp in fp32, unrotating the coded part
//     once ("Differential-KV" README, Flash-Style LSE Combine; "VQKV"
//     summary, 3. Inference Integration, local sliding window of recent
//     tokens kept uncompressed).
//
// Kernels: attn_prep (q rotation, LUT, window partial) -> attn_chunk (code
// streaming, HBM-bound with LDS gathers) -> attn_merge.
#include "kvq_internal.h"

namespace kvq {

// ----------------------------------------------------------- workspace plan
AttnPlan attn_plan(int B, int Hq, int Hkv, int D, int S, int G, int C, int Tc, int W) {
  AttnPlan p{};
  const int SG = S * G;
  const int R = Hq / Hkv;
  p.rp = 0;
  for (int rp = 4; rp >= 1; rp >>= 1) {
    if (rp > R && rp > 1) continue;
    if ((size_t)2 * SG * C * rp * sizeof(float) <= ATTN_LDS_TABLES) { p.rp = rp; break; }
  }
  p.n_hsplit = p.rp ? (R + p.rp - 1) / p.rp : 0;
  if (Tc > 0 && p.rp) {
    const int64_t units = (int64_t)B * Hkv * p.n_hsplit;
    int64_t nc = (256 + units - 1) / units;
    const int64_t min_nc = (Tc + ATTN_MAX_CHUNK - 1) / ATTN_MAX_CHUNK;
    const int64_t max_nc = (Tc + ATTN_MIN_CHUNK - 1) / ATTN_MIN_CHUNK;
    if (nc > max_nc) nc = max_nc;
    if (nc < min_nc) nc = min_nc;
    if (nc < 1) nc = 1;
    p.n_chunks = (int)nc;
    p.chunk = (int)((Tc + nc - 1) / nc);
  } else {
    p.n_chunks = 0;
    p.chunk = 0;
  }
  p.pstride = D + 4;                                    // m, l, pad, pad, o[D]
  p.lut_bytes = (size_t)B * Hq * SG * C * sizeof(float);
  p.part_bytes = (size_t)B * Hq * (p.n_chunks + 1) * p.pstride * sizeof(float);
  p.ws_bytes = ((p.lut_bytes + 255) & ~(size_t)255) + p.part_bytes;
  return p;
}

// -------------------------------------------------------------- attn_prep
// grid (B*Hq), block 256.  q_rot via the in-wave butterfly; LUT (pre-scaled
// by the softmax scale) to the workspace; window partial (m, l, o) in the
// original domain to the last partial slot.
template <int D>
__global__ __launch_bounds__(256) void attn_prep_kernel(
    const float* __restrict__ q, const float* __restrict__ kcb, const uint16_t* __restrict__ kw,
    const uint16_t* __restrict__ vw, float* __restrict__ lut, float* __restrict__ part, int Hq,
    int Hkv, int S, int G, int C, int W, int n_chunks, int pstride, float scale) {
  constexpr int L = D / 8;
  __shared__ float qr[D];
  __shared__ float qo[D];
  __shared__ float sw[256];
  __shared__ float red[8];
  const int bh = blockIdx.x;
  const int b = bh / Hq, h = bh - b * Hq;
  const int kv = h / (Hq / Hkv);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const float* qp = q + (int64_t)bh * D;
  if (tid < 64) {
    const int col = lane % L;
    float v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = qp[col * 8 + i];
    hadamard_row<8, L>(v, lane);
    constexpr float sc = rsqrt_pow2(D);
    if (lane < L) {
#pragma unroll
      for (int i = 0; i < 8; ++i) qr[col * 8 + i] = v[i] * sc;
    }
  }
  for (int d = tid; d < D; d += 256) qo[d] = qp[d];
  __syncthreads();

  // LUT[s][g][c] = scale * sum_j q_rot[g*dsub + j] * C^K_sg[c][j]
  const int dsub = D / G;
  const int SG = S * G;
  float* lp = lut + (int64_t)bh * SG * C;
  for (int i = tid; i < SG * C; i += 256) {
    const int sg = i / C, c = i - sg * C;
    const int g = sg % G;
    const float* cp = kcb + ((int64_t)sg * C + c) * dsub;
    const float* qg = qr + g * dsub;
    float acc = 0.0f;
    for (int j = 0; j < dsub; ++j) acc = __builtin_fmaf(qg[j], cp[j], acc);
    lp[i] = acc * scale;
  }

  // window partial
  float* pp = part + ((int64_t)bh * (n_chunks + 1) + n_chunks) * pstride;
  if (W == 0) {
    if (tid == 0) { pp[0] = -__builtin_inff(); pp[1] = 0.0f; }
    for (int d = tid; d < D; d += 256) pp[4 + d] = 0.0f;
    return;
  }
  const uint16_t* kwp = kw + ((int64_t)b * Hkv + kv) * W * D;
  const uint16_t* vwp = vw + ((int64_t)b * Hkv + kv) * W * D;
  float mloc = -__builtin_inff();
  for (int w0 = 0; w0 < W; w0 += 256) {
    const int w = w0 + tid;
    if (w < W) {
      float acc = 0.0f;
      const uint16_t* kr = kwp + (int64_t)w * D;
      for (int d = 0; d < D; ++d) acc = __builtin_fmaf(qo[d], f16_bits_to_f32(kr[d]), acc);
      acc *= scale;
      mloc = fmaxf(mloc, acc);
    }
  }
  // block max
  float mw = wave_max(mloc);
  if (lane == 0) red[tid >> 6] = mw;
  __syncthreads();
  mw = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  __syncthreads();
  float lsum = 0.0f;
  float oacc = 0.0f;                         // thread d accumulates output dim d (d < D)
  for (int w0 = 0; w0 < W; w0 += 256) {
    const int w = w0 + tid;
    float p = 0.0f;
    if (w < W) {
      float acc = 0.0f;
      const uint16_t* kr = kwp + (int64_t)w * D;
      for (int d = 0; d < D; ++d) acc = __builtin_fmaf(qo[d], f16_bits_to_f32(kr[d]), acc);
      p = __expf(acc * scale - mw);
    }
    lsum += p;
    sw[tid] = p;
    __syncthreads();
    const int nw = (W - w0) < 256 ? (W - w0) : 256;
    for (int d = tid; d < D; d += 256) {
      float a = 0.0f;
      for (int k = 0; k < nw; ++k) a = __builtin_fmaf(sw[k], f16_bits_to_f32(vwp[(int64_t)(w0 + k) * D + d]), a);
      oacc += a;                              // D <= 256: one dim per thread
    }
    __syncthreads();
  }
  float ls = wave_sum(lsum);
  if (lane == 0) red[4 + (tid >> 6)] = ls;
  __syncthreads();
  if (tid == 0) { pp[0] = mw; pp[1] = red[4] + red[5] + red[6] + red[7]; }
  if (tid < D) pp[4 + tid] = oacc;
}

// ------------------------------------------------------------- attn_chunk
// grid (n_chunks, Hkv * n_hsplit, B), block 512.  LDS: LUT and histogram,
// each [SG][C][RP] fp32.  Every thread owns up to CH_TPT tokens of the chunk
// (token = t0 + tid + 512*k), keeps their RP scores in registers across the
// two passes (K scores, then softmax weights and V histogram).
constexpr int CH_THREADS = 512;
constexpr int CH_TPT = ATTN_MAX_CHUNK / CH_THREADS;

template <int RP, int SGC>   // SGC: compile-time S*G (multiple of 16), or 0 = runtime bytes
__global__ __launch_bounds__(CH_THREADS, 1) void attn_chunk_kernel(
    const uint8_t* __restrict__ kcodes, const uint8_t* __restrict__ vcodes,
    const float* __restrict__ vcb, const float* __restrict__ lut, float* __restrict__ part,
    int Hq, int Hkv, int D, int S, int G, int C, int Tc, int n_chunks, int chunk, int n_hsplit,
    int pstride) {
  extern __shared__ __attribute__((aligned(16))) float sm[];
  const int SG = SGC ? SGC : S * G;
  const int tabn = SG * C * RP;
  float* tl = sm;                       // LUT   [SG][C][RP]
  float* th = sm + tabn;                // hist  [SG][C][RP]
  __shared__ float red[16][RP];
  __shared__ float mx[RP], lt[RP];

  const int ci = blockIdx.x;
  const int kvs = blockIdx.y;
  const int b = blockIdx.z;
  const int kv = kvs / n_hsplit;
  const int hs = kvs - kv * n_hsplit;
  const int R = Hq / Hkv;
  const int h0 = kv * R + hs * RP;                      // first query head of this block
  const int nh = (R - hs * RP) < RP ? (R - hs * RP) : RP; // real heads in this block
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int t0 = ci * chunk;
  const int t1 = (t0 + chunk) < Tc ? (t0 + chunk) : Tc;

  // ---- tables
  for (int i = tid; i < SG * C; i += CH_THREADS) {
#pragma unroll
    for (int r = 0; r < RP; ++r) {
      const int hr = h0 + (r < nh ? r : nh - 1);
      tl[i * RP + r] = lut[((int64_t)b * Hq + hr) * SG * C + i];
      th[i * RP + r] = 0.0f;
    }
  }
  __syncthreads();

  const int64_t rowbase = ((int64_t)b * Hkv + kv) * (int64_t)Tc;
  float sc[CH_TPT][RP];
  // ---- pass 1: K scores
#pragma unroll
  for (int k = 0; k < CH_TPT; ++k) {
    const int t = t0 + tid + CH_THREADS * k;
#pragma unroll
    for (int r = 0; r < RP; ++r) sc[k][r] = -__builtin_inff();
    if (t < t1) {
      float acc[RP];
#pragma unroll
      for (int r = 0; r < RP; ++r) acc[r] = 0.0f;
      const uint8_t* row = kcodes + (rowbase + t) * SG;
      if constexpr (SGC != 0) {
#pragma unroll
        for (int w4 = 0; w4 < SGC / 16; ++w4) {
          const uint4 wv = reinterpret_cast<const uint4*>(row)[w4];
          const uint32_t ws[4] = {wv.x, wv.y, wv.z, wv.w};
#pragma unroll
          for (int q = 0; q < 4; ++q) {
#pragma unroll
            for (int by = 0; by < 4; ++by) {
              const int sg = w4 * 16 + q * 4 + by;
              int z = (ws[q] >> (8 * by)) & 255;
              z = z < C ? z : C - 1;
              const float* e = tl + (sg * C + z) * RP;
              if constexpr (RP == 4) {
                const float4 v = *reinterpret_cast<const float4*>(e);
                acc[0] += v.x; acc[1] += v.y; acc[2] += v.z; acc[3] += v.w;
              } else if constexpr (RP == 2) {
                const float2 v = *reinterpret_cast<const float2*>(e);
                acc[0] += v.x; acc[1] += v.y;
              } else {
                acc[0] += e[0];
              }
            }
          }
        }
      } else {
        for (int sg = 0; sg < SG; ++sg) {
          int z = row[sg];
          z = z < C ? z : C - 1;
          const float* e = tl + (sg * C + z) * RP;
#pragma unroll
          for (int r = 0; r < RP; ++r) acc[r] += e[r];
        }
      }
#pragma unroll
      for (int r = 0; r < RP; ++r) sc[k][r] = acc[r];
    }
  }
  // ---- chunk max per head
  float m[RP];
#pragma unroll
  for (int r = 0; r < RP; ++r) {
    float v = -__builtin_inff();
#pragma unroll
    for (int k = 0; k < CH_TPT; ++k) v = fmaxf(v, sc[k][r]);
    v = wave_max(v);
    if (lane == 0) red[wave][r] = v;
  }
  __syncthreads();
  if (tid < RP) {
    float v = red[0][tid];
    for (int w = 1; w < CH_THREADS / 64; ++w) v = fmaxf(v, red[w][tid]);
    mx[tid] = v;
  }
  __syncthreads();
#pragma unroll
  for (int r = 0; r < RP; ++r) m[r] = mx[r];

  // ---- pass 2: weights, V histogram
  float ls[RP];
#pragma unroll
  for (int r = 0; r < RP; ++r) ls[r] = 0.0f;
#pragma unroll
  for (int k = 0; k < CH_TPT; ++k) {
    const int t = t0 + tid + CH_THREADS * k;
    if (t < t1) {
      float p[RP];
#pragma unroll
      for (int r = 0; r < RP; ++r) { p[r] = __expf(sc[k][r] - m[r]); ls[r] += p[r]; }
      const uint8_t* row = vcodes + (rowbase + t) * SG;
      if constexpr (SGC != 0) {
#pragma unroll
        for (int w4 = 0; w4 < SGC / 16; ++w4) {
          const uint4 wv = reinterpret_cast<const uint4*>(row)[w4];
          const uint32_t ws[4] = {wv.x, wv.y, wv.z, wv.w};
#pragma unroll
          for (int q = 0; q < 4; ++q) {
#pragma unroll
            for (int by = 0; by < 4; ++by) {
              const int sg = w4 * 16 + q * 4 + by;
              int z = (ws[q] >> (8 * by)) & 255;
              z = z < C ? z : C - 1;
              float* e = th + (sg * C + z) * RP;
#pragma unroll
              for (int r = 0; r < RP; ++r) atomicAdd(e + r, p[r]);
            }
          }
        }
      } else {
        for (int sg = 0; sg < SG; ++sg) {
          int z = row[sg];
          z = z < C ? z : C - 1;
          float* e = th + (sg * C + z) * RP;
#pragma unroll
          for (int r = 0; r < RP; ++r) atomicAdd(e + r, p[r]);
        }
      }
    }
  }
#pragma unroll
  for (int r = 0; r < RP; ++r) {
    const float v = wave_sum(ls[r]);
    if (lane == 0) red[8 + wave][r] = v;   // rows 8..15 (max rows no longer needed)
  }
  __syncthreads();
  if (tid < RP) {
    float v = 0.0f;
    for (int w = 0; w < CH_THREADS / 64; ++w) v += red[8 + w][tid];
    lt[tid] = v;
  }
  __syncthreads();

  // ---- o_rot[r][d] = sum_s sum_c W[s][g(d)][c][r] * C^V[s][g][c][j]
  const int dsub = D / G;
  for (int o = tid; o < RP * D; o += CH_THREADS) {
    const int r = o / D, d = o - r * D;
    if (r >= nh) continue;
    const int g = d / dsub, j = d - g * dsub;
    float acc = 0.0f;
    for (int s = 0; s < S; ++s) {
      const int sg = s * G + g;
      const float* cp = vcb + ((int64_t)sg * C) * dsub + j;
      const float* hp = th + (sg * C) * RP + r;
#pragma unroll 8
      for (int c = 0; c < C; ++c) acc = __builtin_fmaf(hp[c * RP], cp[(int64_t)c * dsub], acc);
    }
    float* pp = part + ((int64_t)(b * Hq + h0 + r) * (n_chunks + 1) + ci) * pstride;
    pp[4 + d] = acc;
    if (d == 0) { pp[0] = mx[r]; pp[1] = lt[r]; }
  }
}

// ------------------------------------------------------------- attn_merge
// grid (B*Hq), block 64.  out = (H * sum_i w_i o_rot_i + w_win o_win) /
// (sum_i w_i l_i + w_win l_win), w = exp(m - m*).
template <int D>
__global__ __launch_bounds__(64) void attn_merge_kernel(const float* __restrict__ part,
                                                        float* __restrict__ out, int n_chunks,
                                                        int pstride) {
  constexpr int L = D / 8;
  const int bh = blockIdx.x;
  const int lane = threadIdx.x;
  const float* pb = part + (int64_t)bh * (n_chunks + 1) * pstride;
  float mloc = -__builtin_inff();
  for (int i = lane; i <= n_chunks; i += 64) mloc = fmaxf(mloc, pb[(int64_t)i * pstride]);
  const float ms = wave_max(mloc);
  const int col = lane % L;
  float acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.0f;
  float den = 0.0f;
  for (int i = 0; i < n_chunks; ++i) {
    const float* pi = pb + (int64_t)i * pstride;
    const float mi = pi[0];
    if (mi == -__builtin_inff()) continue;
    const float wgt = __expf(mi - ms);
    den = __builtin_fmaf(wgt, pi[1], den);
    const float4* o4 = reinterpret_cast<const float4*>(pi + 4 + col * 8);
    const float4 a = o4[0], c = o4[1];
    acc[0] = __builtin_fmaf(wgt, a.x, acc[0]); acc[1] = __builtin_fmaf(wgt, a.y, acc[1]);
    acc[2] = __builtin_fmaf(wgt, a.z, acc[2]); acc[3] = __builtin_fmaf(wgt, a.w, acc[3]);
    acc[4] = __builtin_fmaf(wgt, c.x, acc[4]); acc[5] = __builtin_fmaf(wgt, c.y, acc[5]);
    acc[6] = __builtin_fmaf(wgt, c.z, acc[6]); acc[7] = __builtin_fmaf(wgt, c.w, acc[7]);
  }
  hadamard_row<8, L>(acc, lane);
  constexpr float sc = rsqrt_pow2(D);
  const float* pw = pb + (int64_t)n_chunks * pstride;
  const float mw = pw[0];
  const float ww = mw == -__builtin_inff() ? 0.0f : __expf(mw - ms);
  den = __builtin_fmaf(ww, pw[1], den);
  const float inv = 1.0f / den;
  if (lane < L) {
    const float4* o4 = reinterpret_cast<const float4*>(pw + 4 + col * 8);
    const float4 a = o4[0], c = o4[1];
    const float wv[8] = {a.x, a.y, a.z, a.w, c.x, c.y, c.z, c.w};
    float r[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) r[e] = (acc[e] * sc + ww * wv[e]) * inv;
    float4* op = reinterpret_cast<float4*>(out + (int64_t)bh * D + col * 8);
    op[0] = make_float4(r[0], r[1], r[2], r[3]);
    op[1] = make_float4(r[4], r[5], r[6], r[7]);
  }
}

// --------------------------------------------------------------- launcher
template <int RP>
static hipError_t launch_chunk_rp(const AttnPlan& p, int SG, const uint8_t* kc, const uint8_t* vc,
                                  const float* vcb, const float* lut, float* part, int B, int Hq,
                                  int Hkv, int D, int S, int G, int C, int Tc, hipStream_t st) {
  dim3 grid(p.n_chunks, Hkv * p.n_hsplit, B);
  const size_t lds = (size_t)2 * SG * C * RP * sizeof(float);
#define KVQ_CH(SGV)                                                                            \
  {                                                                                            \
    auto kern = attn_chunk_kernel<RP, SGV>;                                                    \
    hipError_t e = hipFuncSetAttribute((const void*)kern,                                      \
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);  \
    if (e != hipSuccess) return e;                                                             \
    kern<<<grid, CH_THREADS, lds, st>>>(kc, vc, vcb, lut, part, Hq, Hkv, D, S, G, C, Tc,       \
                                        p.n_chunks, p.chunk, p.n_hsplit, p.pstride);           \
    return hipGetLastError();                                                                  \
  }
  if (SG == 16) KVQ_CH(16)
  if (SG == 32) KVQ_CH(32)
  if (SG == 64) KVQ_CH(64)
  KVQ_CH(0)
#undef KVQ_CH
}

hipError_t launch_attend(const AttnPlan& p, int B, int Hq, int Hkv, int D, int S, int G, int C,
                         int Tc, int W, float scale, const float* q, const uint8_t* kc,
                         const uint8_t* vc, const float* kcb, const float* vcb,
                         const uint16_t* kw, const uint16_t* vw, float* out, void* ws,
                         hipStream_t st) {
  float* lut = reinterpret_cast<float*>(ws);
  float* part = reinterpret_cast<float*>(reinterpret_cast<uint8_t*>(ws) +
                                         ((p.lut_bytes + 255) & ~(size_t)255));
  const int SG = S * G;
#define KVQ_PREP(DD)                                                                          \
  attn_prep_kernel<DD><<<dim3(B * Hq), 256, 0, st>>>(q, kcb, kw, vw, lut, part, Hq, Hkv, S, G,  \
                                                     C, W, p.n_chunks, p.pstride, scale);
  if (D == 64) { KVQ_PREP(64) } else if (D == 128) { KVQ_PREP(128) } else { KVQ_PREP(256) }
#undef KVQ_PREP
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (p.n_chunks > 0) {
    if (p.rp == 4) e = launch_chunk_rp<4>(p, SG, kc, vc, vcb, lut, part, B, Hq, Hkv, D, S, G, C, Tc, st);
    else if (p.rp == 2) e = launch_chunk_rp<2>(p, SG, kc, vc, vcb, lut, part, B, Hq, Hkv, D, S, G, C, Tc, st);
    else e = launch_chunk_rp<1>(p, SG, kc, vc, vcb, lut, part, B, Hq, Hkv, D, S, G, C, Tc, st);
    if (e != hipSuccess) return e;
  }
  if (D == 64) attn_merge_kernel<64><<<dim3(B * Hq), 64, 0, st>>>(part, out, p.n_chunks, p.pstride);
  else if (D == 128) attn_merge_kernel<128><<<dim3(B * Hq), 64, 0, st>>>(part, out, p.n_chunks, p.pstride);
  else attn_merge_kernel<256><<<dim3(B * Hq), 64, 0, st>>>(part, out, p.n_chunks, p.pstride);
  return hipGetLastError();
}

}  // namespace kvq
