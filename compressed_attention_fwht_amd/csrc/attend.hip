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
//     fp32 partial (m, l, o_rot).  The dense fp16 window enters the same
//     partials with its V rows rotated like the codebooks (H v / sqrt(D)): a
//     short window as one slice per chunk block, folded into the chunk's
//     record; a long one as blocks of its own in the same grid.  The merge
//     kernel combines the partials by log-sum-exp in fp32 and unrotates once
//     ("Differential-KV" README, Flash-Style LSE Combine; "VQKV" summary,
//     3. Inference Integration, local sliding window of recent tokens kept
//     uncompressed).
//
// Kernels: [attn_lut (q rotation slices, LUT)] -> attn_chunk (LUT when not
// staged from attn_lut, code streaming, K scores, V histogram, contraction,
// window) -> attn_merge (LSE merge, unrotation).
//
// The histogram accumulates the weights p = exp(s - m_chunk) in [0, 1] as
// fixed-point integers round(p * 2^F) with LDS integer atomics (ds_add_u32,
// or ds_add_u64 carrying two heads' 32-bit fields at once): on gfx950 LDS
// float atomics retire an order of magnitude slower than integer ones.
// F = 31 - ceil(log2(l)) per head, l = sum_t p_t of the chunk (at least 1),
// keeps every bin and every field sum below 2^32, so packed fields never
// carry into each other, and bounds the weight rounded away per token by
// l * 2^-32, so the rounding error of the chunk stays below chunk * 2^-32 of
// l even when one token dominates.  The chunk's l is the sum of the same
// integers, so numerator and denominator see the same rounded weights.
#include "attend_common.h"

namespace kvq {

static int ceil_log2(int64_t v) {
  int k = 0;
  while (((int64_t)1 << k) < v) ++k;
  return k;
}

// ----------------------------------------------------------- workspace plan
// V histogram: per sg a block of C * RP 32-bit words plus a 4-word pad
constexpr int HIST_PAD = 4;
__host__ __device__ constexpr int hist_stride(int C, int RP) { return C * RP + HIST_PAD; }

AttnPlan attn_plan(int B, int Hq, int Hkv, int D, int S, int G, int C, int Tc, int W) {
  AttnPlan p{};
  const int SG = S * G;
  const int R = Hq / Hkv;
  if (attn_rc_eligible(D, G, S, C, Hq, Hkv, Tc)) {
    // rotated-code kernels: four query heads per block, one chunk of at most
    // RC_MAX_CHUNK tokens per block, about 256 blocks; the window as a slice
    // of each chunk block, or in short blocks of the LUT kernel's grid when
    // the slices would be long
    p.rc = 1;
    p.rp = 4;
    p.n_hsplit = (R + 3) / 4;
    const int64_t units = (int64_t)B * Hkv * p.n_hsplit;
    int64_t nc = (256 + units - 1) / units;
    const int64_t min_nc = (Tc + RC_MAX_CHUNK - 1) / RC_MAX_CHUNK;
    const int64_t max_nc = (Tc + ATTN_MIN_CHUNK - 1) / ATTN_MIN_CHUNK;
    if (nc > max_nc) nc = max_nc;
    if (nc < min_nc) nc = min_nc;
    if (nc < 1) nc = 1;
    p.chunk = (int)((Tc + nc - 1) / nc);
    p.n_chunks = (int)((Tc + p.chunk - 1) / p.chunk);
    p.wslice = attn_rc_window_slice(W, p.n_chunks);
    p.n_wblocks = W > 0 && p.wslice == 0 ? attn_rc_window_blocks(W) : 0;
    p.pstride = D + 4;
    p.lut_slice = attn_rc_table_bytes(S, G);
    // per-unit LUT segments, then the V codebook in the contraction's order
    p.lut_bytes = (size_t)units * p.lut_slice + (size_t)S * G * C * (D / G) * sizeof(float);
    p.part_bytes = (size_t)B * Hq * (p.n_chunks + p.n_wblocks) * p.pstride * sizeof(float);
    p.ws_bytes = ((p.lut_bytes + 255) & ~(size_t)255) + p.part_bytes;
    return p;
  }
  // codeword ranges per (stage, 4-dim) item of the V contraction: aim at 512
  // items (at most 16 ranges), fewer when LDS is short; more heads per block
  // win over more ranges
  int P0 = 512 / (S * (D / 4));
  if (P0 < 1) P0 = 1;
  if (P0 > 16) P0 = 16;
  p.rp = 0;
  for (int rp = 4; rp >= 1 && !p.rp; rp >>= 1) {
    if (rp > R && rp > 1) continue;
    const size_t tab = (size_t)SG * hist_stride(C, rp) * 4;
    for (int P = P0; P >= 1; P >>= 1) {
      if (tab + (size_t)S * P * rp * D * 4 <= ATTN_LDS_TABLES) { p.rp = rp; p.cparts = P; break; }
    }
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
    p.chunk = (int)((Tc + nc - 1) / nc);
    p.n_chunks = (int)((Tc + p.chunk - 1) / p.chunk);   // no empty trailing chunk
  }
  if (Tc == 0) {                                        // window only: no tables needed
    p.rp = R >= 4 ? 4 : R >= 2 ? 2 : 1;
    p.n_hsplit = (R + p.rp - 1) / p.rp;
    p.cparts = 1;
  }
  // window: a slice of at most 4096/D tokens on each chunk block (one token
  // per row of D/8 lanes; its row sums need 8*RP*D floats of LDS beside the
  // LUT), else blocks of its own of ATTN_WIN_BLOCK tokens
  p.wslice = p.n_wblocks = 0;
  if (W > 0) {
    const int per = p.n_chunks > 0 ? (W + p.n_chunks - 1) / p.n_chunks : 0;
    const int sp = S * p.cparts > 8 ? S * p.cparts : 8;
    if (p.n_chunks > 0 && per <= 4096 / D &&
        (size_t)SG * hist_stride(C, p.rp) * 4 + (size_t)sp * p.rp * D * 4 <= ATTN_LDS_TABLES)
      p.wslice = per;
    else
      p.n_wblocks = (W + ATTN_WIN_BLOCK - 1) / ATTN_WIN_BLOCK;
  }
  // LUT built by the chunk blocks themselves unless the K codebook re-reads
  // (S*C*D floats per block, from L2) outweigh one LUT pass
  p.fuse_lut = p.n_chunks > 0 &&
               (size_t)B * Hkv * p.n_hsplit * p.n_chunks * S * C * D * 4 <= ((size_t)96 << 20);
  p.pstride = D + 4;                                    // m, l, pad, pad, o[D]
  p.lut_slice = ((size_t)SG * C * (p.rp ? p.rp : 1) * 4 + 255) & ~(size_t)255;
  p.lut_bytes = p.n_chunks && !p.fuse_lut ? (size_t)B * Hkv * p.n_hsplit * p.lut_slice : 0;
  p.part_bytes = (size_t)B * Hq * (p.n_chunks + p.n_wblocks) * p.pstride * sizeof(float);
  p.ws_bytes = ((p.lut_bytes + 255) & ~(size_t)255) + p.part_bytes;
  return p;
}

// --------------------------------------------------------------- attn_lut
// grid (B*Hkv*n_hsplit, S*G), block 256.  Block (unit, sg) writes the LUT
// entries of one (s, g) table for the RP query heads of its unit, laid out
// [unit][sg][c][RP] so a chunk block stages its whole table with contiguous
// copies.  Heads past the group's last one repeat it (never read back).
template <int RP, int D>
__global__ __launch_bounds__(256) void attn_lut_kernel(const float* __restrict__ q,
                                                       const float* __restrict__ kcb,
                                                       float* __restrict__ lut, int Hq, int Hkv,
                                                       int n_hsplit, int G, int C,
                                                       size_t lut_slice, float scale,
                                                       const float* __restrict__ ksm,
                                                       int64_t ksm_rows) {
  constexpr int L = D / 8;                 // lanes per query row in the butterfly
  constexpr int ROWS = 64 / L;             // query rows per wave
  __shared__ float qs[RP][D];
  const int unit = blockIdx.x, sg = blockIdx.y;
  const int hs = unit % n_hsplit;
  const int bkv = unit / n_hsplit;
  const int kv = bkv % Hkv, b = bkv / Hkv;
  const int R = Hq / Hkv;
  const int nh = (R - hs * RP) < RP ? (R - hs * RP) : RP;
  const int g = sg % G, dsub = D / G;
  const int tid = threadIdx.x, lane = tid & 63;
  // scale * H_D q for the RP heads: wave 0, L lanes x 8 elements per row
  if (tid < 64) {
#pragma unroll
    for (int r0 = 0; r0 < RP; r0 += ROWS) {
      const int r = r0 + lane / L;
      const int rr = r < RP ? r : RP - 1;
      const int h = kv * R + hs * RP + (rr < nh ? rr : nh - 1);
      const float* qp = q + ((int64_t)b * Hq + h) * D + (lane % L) * 8;
      float v[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = qp[e];
      if (ksm != nullptr) smooth_query<D>(v, ksm, b, kv, Hkv, ksm_rows, lane % L);
      hadamard_row<8, L>(v, lane);
      const float rs = scale * rsqrt_pow2(D);
      if (r < RP) {
#pragma unroll
        for (int e = 0; e < 8; ++e) qs[r][(lane % L) * 8 + e] = v[e] * rs;
      }
    }
  }
  __syncthreads();
  float* dst = reinterpret_cast<float*>(reinterpret_cast<uint8_t*>(lut) + unit * lut_slice) +
               (size_t)sg * C * RP;
  for (int c = tid; c < C; c += 256) {
    const float* cp = kcb + ((int64_t)sg * C + c) * dsub;
    float acc[RP];
#pragma unroll
    for (int r = 0; r < RP; ++r) acc[r] = 0.0f;
    for (int j = 0; j < dsub; ++j) {
      const float cv = cp[j];
#pragma unroll
      for (int r = 0; r < RP; ++r) acc[r] = __builtin_fmaf(qs[r][g * dsub + j], cv, acc[r]);
    }
#pragma unroll
    for (int r = 0; r < RP; ++r) dst[c * RP + r] = acc[r];
  }
}

// ------------------------------------------------------------- attn_chunk
// grid (n_chunks + n_wblocks, Hkv * n_hsplit, B), block 512.  A short
// window rides on the chunk blocks (a slice each, win_slice_*); a long one gets
// blocks x >= n_chunks of its own (window_partial).  LDS: one table region
// that holds the LUT ([S*G][C][RP] floats) during pass 1 and the weight
// histogram (integers, layout below) during pass 2, plus the contraction's
// partial sums.  Each thread owns up to CH_TPT tokens of the chunk
// (token = t0 + tid + 512*k) and keeps their RP scores in registers across
// the two passes.
constexpr int CH_THREADS = 512;
constexpr int CH_TPT = ATTN_MAX_CHUNK / CH_THREADS;

// Histogram layout: per sg a block of HIST_PAD + C * RP 32-bit words holding
// [RP/2][C] 64-bit bins (the two 32-bit weights of a head pair in one bin),
// or [C] 32-bit ones for RP = 1.  Pair-major keeps the bins of one atomic
// instruction (same sg and pair, random z) 8 bytes apart, so they spread over
// twice the LDS banks a [C][RP] layout reaches; the 4-word pad per block
// puts the blocks of different sg on different banks, which the contraction
// (lanes of one wave on different groups, same codeword) reads together.

template <int RP>
__device__ __forceinline__ void hist_add(uint32_t* tab, int sg, int z, int C,
                                         const uint32_t (&pw)[RP]) {
  uint32_t* blk = tab + sg * hist_stride(C, RP);
  if constexpr (RP == 1) {
    atomicAdd(blk + z, pw[0]);
  } else {
    unsigned long long* t64 = reinterpret_cast<unsigned long long*>(blk);
#pragma unroll
    for (int r = 0; r < RP; r += 2)
      atomicAdd(t64 + (r / 2) * C + z,
                (unsigned long long)pw[r] | ((unsigned long long)pw[r + 1] << 32));
  }
}

// bin of head r, codeword c inside one sg's block
template <int RP>
__device__ __forceinline__ int hist_bin(int c, int r, int C) {
  if constexpr (RP == 1) return c;
  else return ((r >> 1) * C + c) * 2 + (r & 1);
}

template <int RP>
__device__ __forceinline__ void lut_add(const float* tab, int e, float (&acc)[RP]) {
  if constexpr (RP == 4) {
    const float4 v = *reinterpret_cast<const float4*>(tab + e);
    acc[0] += v.x; acc[1] += v.y; acc[2] += v.z; acc[3] += v.w;
  } else if constexpr (RP == 2) {
    const float2 v = *reinterpret_cast<const float2*>(tab + e);
    acc[0] += v.x; acc[1] += v.y;
  } else {
    acc[0] += tab[e];
  }
}

// Visit the S*G code bytes of one token row: f(sg, z) with z clamped below C.
template <int SGC, typename Fn>
__device__ __forceinline__ void for_codes(const uint8_t* row, int SG, int C, Fn&& f) {
  if constexpr (SGC != 0) {
#pragma unroll
    for (int w4 = 0; w4 < SGC / 16; ++w4) {
      const uint4 wv = reinterpret_cast<const uint4*>(row)[w4];
      const uint32_t ws[4] = {wv.x, wv.y, wv.z, wv.w};
#pragma unroll
      for (int qd = 0; qd < 4; ++qd) {
#pragma unroll
        for (int by = 0; by < 4; ++by) {
          int z = (ws[qd] >> (8 * by)) & 255;
          if (C < 256) z = z < C ? z : C - 1;
          f(w4 * 16 + qd * 4 + by, z);
        }
      }
    }
  } else {
    for (int sg = 0; sg < SG; ++sg) {
      int z = row[sg];
      z = z < C ? z : C - 1;
      f(sg, z);
    }
  }
}

// Register-staged code rows (compile-time S*G only): load_codes issues the
// 16-byte loads of one token row, visit_codes walks the bytes like for_codes.
template <int SGC>
__device__ __forceinline__ void load_codes(const uint8_t* row, uint4 (&w)[SGC / 16]) {
#pragma unroll
  for (int i = 0; i < SGC / 16; ++i) w[i] = reinterpret_cast<const uint4*>(row)[i];
}

template <int SGC, typename Fn>
__device__ __forceinline__ void visit_codes(const uint4 (&w)[SGC / 16], int C, Fn&& f) {
#pragma unroll
  for (int w4 = 0; w4 < SGC / 16; ++w4) {
    const uint32_t ws[4] = {w[w4].x, w[w4].y, w[w4].z, w[w4].w};
#pragma unroll
    for (int qd = 0; qd < 4; ++qd) {
#pragma unroll
      for (int by = 0; by < 4; ++by) {
        int z = (ws[qd] >> (8 * by)) & 255;
        if (C < 256) z = z < C ? z : C - 1;
        f(w4 * 16 + qd * 4 + by, z);
      }
    }
  }
}

// Window slice riding on a chunk block: up to 4096/D tokens, one per token
// row of L = D/8 lanes.  The K row, the V row and q are loaded when the block
// starts (their latency overlaps the LUT staging) and the scores are formed
// once they have landed.  The slice keeps a softmax partial of its own (own
// max, float weights, V rotated like the codebooks) whose reductions share
// the chunk's barriers, and is folded into the chunk's record at the end; a
// common fixed-point scale would round every chunk token against a window
// maximum that may dwarf it.  Returns whether this row holds a token.
// The loads are issued whatever the slice holds (rows past it read the last
// window row, or, with no window at all, the first bytes of q) so the number
// of loads in flight is fixed and later waits count exactly; rows without a
// token come back as zeros.
template <int RP, int D>
__device__ __forceinline__ bool win_slice_load(uint4& kraw, uint4& vraw, float (&qv)[RP][8],
                                               const float* __restrict__ q,
                                               const uint16_t* __restrict__ kw,
                                               const uint16_t* __restrict__ vw, bool have,
                                               int b, int kv, int h0, int nh, int Hq, int Hkv,
                                               int wstride, int wa, int wb, int tid) {
  constexpr int L = D / 8;
  const int row = tid / L, col = tid % L;
  const int t = wa + row;
  const bool act = have && t < wb;
  const int tl = t < wb ? t : (wb > 0 ? wb - 1 : 0);
  const uint16_t* kp = reinterpret_cast<const uint16_t*>(q) + col * 8;
  const uint16_t* vp = kp;
  if (have) {
    const int64_t off = (((int64_t)b * Hkv + kv) * wstride + tl) * D + col * 8;
    kp = kw + off;
    vp = vw + off;
  }
  const uint4 kl = *reinterpret_cast<const uint4*>(kp);
  const uint4 vl = *reinterpret_cast<const uint4*>(vp);
  const uint4 z = make_uint4(0u, 0u, 0u, 0u);
  kraw = act ? kl : z;
  vraw = act ? vl : z;
#pragma unroll
  for (int r = 0; r < RP; ++r) {
    const float4* qp = reinterpret_cast<const float4*>(
        q + ((int64_t)b * Hq + h0 + (r < nh ? r : nh - 1)) * D + col * 8);
    const float4 x0 = qp[0], x1 = qp[1];
    qv[r][0] = x0.x; qv[r][1] = x0.y; qv[r][2] = x0.z; qv[r][3] = x0.w;
    qv[r][4] = x1.x; qv[r][5] = x1.y; qv[r][6] = x1.z; qv[r][7] = x1.w;
  }
  return act;
}

template <int RP, int D>
__device__ __forceinline__ void win_slice_scores(float (&sw)[RP], uint4 kraw,
                                                 const float (&qv)[RP][8], bool act,
                                                 float scale) {
  constexpr int L = D / 8;
  const uint32_t kr[4] = {kraw.x, kraw.y, kraw.z, kraw.w};
  float kx[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    kx[2 * i] = f16_bits_to_f32(kr[i]);
    kx[2 * i + 1] = f16_bits_to_f32(kr[i] >> 16);
  }
#pragma unroll
  for (int r = 0; r < RP; ++r) {
    float dot = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) dot = __builtin_fmaf(qv[r][e], kx[e], dot);
    dot = row_sum<L>(dot) * scale;
    sw[r] = act ? dot : -__builtin_inff();
  }
}

// SGC: compile-time S*G (multiple of 16), or 0 = runtime bytes.  FUSE: the
// block builds its unit's LUT itself (else it stages the one attn_lut_kernel
// wrote); separate instances keep each path's memory waits exact.
// wslice > 0: block ci also owns window tokens [ci*wslice, (ci+1)*wslice),
// folded into its record; otherwise blocks x >= n_chunks are window blocks.
template <int RP, int SGC, int D, bool FUSE>
__global__ __launch_bounds__(CH_THREADS, 1) void attn_chunk_kernel(
    const uint8_t* __restrict__ kcodes, const uint8_t* __restrict__ vcodes,
    const float* __restrict__ vcb, const float* __restrict__ lut, float* __restrict__ part,
    int Hq, int Hkv, int S, int G, int C, int Tc, int n_chunks, int chunk, int n_hsplit,
    int pstride, int cparts, size_t lut_slice, const float* __restrict__ kcb,
    const float* __restrict__ q,
    const uint16_t* __restrict__ kw, const uint16_t* __restrict__ vw, int W, int wslice,
    int nslots, float scale, int cstride, int wstride, const float* __restrict__ ksm,
    int64_t ksm_rows) {
  constexpr int L = D / 8;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int ci = blockIdx.x;
  const int unit = blockIdx.y;                          // kv * n_hsplit + hs
  const int b = blockIdx.z;
  const int kv = unit / n_hsplit, hs = unit - kv * n_hsplit;
  const int R = Hq / Hkv;
  const int h0 = kv * R + hs * RP;
  const int nh = (R - hs * RP) < RP ? (R - hs * RP) : RP;
  if (ci >= n_chunks) {                                 // window block (uniform per block)
    const int w0 = (ci - n_chunks) * ATTN_WIN_BLOCK;
    const int w1 = (w0 + ATTN_WIN_BLOCK) < W ? (w0 + ATTN_WIN_BLOCK) : W;
    window_partial<RP, D>(q, kw, vw, part, smem, b, kv, h0, nh, Hq, Hkv, wstride, w0, w1, ci,
                          nslots, pstride, scale);
    return;
  }
  const int SG = SGC ? SGC : S * G;
  const int tabn = SG * C * RP;                         // LUT entries
  const int tabh = SG * hist_stride(C, RP);             // histogram words (the region's size)
  float* tabf = reinterpret_cast<float*>(smem);         // LUT during pass 1
  uint32_t* tabu = reinterpret_cast<uint32_t*>(smem);   // histogram during pass 2
  float* cpart = reinterpret_cast<float*>(smem + (((size_t)tabh * 4 + 15) & ~(size_t)15));
  __shared__ float red_f[8][RP], red_wf[8][RP], red_wl[8][RP], red_l[8][RP];
  __shared__ uint32_t red_u[8][RP];
  __shared__ float mx[RP], mxw[RP], ltw[RP];
  __shared__ uint32_t lt[RP];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int t0 = ci * chunk;
  const int t1 = (t0 + chunk) < Tc ? (t0 + chunk) : Tc;

  const int64_t rowbase = ((int64_t)b * Hkv + kv) * (int64_t)cstride;
  // The first KP token rows of K codes (and of V codes) are staged in
  // registers (32 VGPRs each) so their HBM latency overlaps the LUT work.
  // Prefetches are issued unconditionally, rows past the chunk clamped to its
  // last one: vector loads complete in order, and a load that may or may not
  // have been issued makes later waits drain everything in flight.  A block
  // that builds its LUT issues its K and V rows right after the query and
  // codebook loads the table needs; one that stages a prepared LUT issues its
  // K rows first and waits for all its loads once (the LDS copy), so its V
  // rows follow pass 1 instead.
  constexpr int SGW = SGC ? SGC / 16 : 1;
  constexpr int KP = SGC ? (128 / SGC < CH_TPT ? 128 / SGC : CH_TPT) : 0;
  constexpr int KPA = KP ? KP : 1;
  uint4 cpre[KPA][SGW], vpre[KPA][SGW];
  auto prefetch_rows = [&](const uint8_t* __restrict__ codes_, uint4 (&dst)[KPA][SGW]) {
    if constexpr (KP > 0) {
#pragma unroll
      for (int k = 0; k < KP; ++k) {
        const int t = t0 + tid + CH_THREADS * k;
        load_codes<SGC>(codes_ + (rowbase + (t < t1 ? t : t1 - 1)) * SG, dst[k]);
      }
    }
  };
  if constexpr (!FUSE) prefetch_rows(kcodes, cpre);

  if constexpr (FUSE) {
    // ---- build this unit's LUT in LDS: scale * H q / sqrt(D) for the RP
    // heads, then entry (sg, c) = q_rot_g . C^K_sg[c], summed in the order
    // attn_lut_kernel uses.  For dsub = 8 and C = 256 a thread owns one sg
    // per pass (16 * pass + tid / 32) and the codewords c = tid % 32 + 32 k,
    // k < 8: its slice of q_rot is read from LDS once per pass, and a wave's
    // row loads stay two contiguous 1 KiB runs.  The pass's rows come in two
    // halves of 4 (both in flight across the q rotation), each half of the
    // next pass issued across the arithmetic of the current one.
    __shared__ float qs[RP][D];
    constexpr int QROWS = 64 / L;                       // q rows per wave-wide load
    constexpr int QIT = (RP + QROWS - 1) / QROWS;
    float qraw[QIT][8];
#pragma unroll
    for (int i = 0; i < QIT; ++i) {
      const int r = i * QROWS + lane / L;
      const int rr = r < RP ? r : RP - 1;
      const float4* qp = reinterpret_cast<const float4*>(
          q + ((int64_t)b * Hq + h0 + (rr < nh ? rr : nh - 1)) * D + (lane % L) * 8);
      const float4 x0 = qp[0], x1 = qp[1];
      qraw[i][0] = x0.x; qraw[i][1] = x0.y; qraw[i][2] = x0.z; qraw[i][3] = x0.w;
      qraw[i][4] = x1.x; qraw[i][5] = x1.y; qraw[i][6] = x1.z; qraw[i][7] = x1.w;
    }
    const int dsub = D / G;
    const int nit = SG * C;
    const bool fast = dsub == 8 && C == 256;
    const int npass = (SG + 15) / 16;
    float4 cb0[4][2], cb1[4][2];
    auto load_half = [&](float4 (&cb)[4][2], int pass, int half) {   // rows past nit: the last
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int it = (16 * pass + tid / 32) * 256 + tid % 32 + 32 * (half * 4 + i);
        const float4* cp = reinterpret_cast<const float4*>(kcb + (int64_t)(it < nit ? it : nit - 1) * 8);
        cb[i][0] = cp[0];
        cb[i][1] = cp[1];
      }
    };
    if (fast) {
      load_half(cb0, 0, 0);
      load_half(cb1, 0, 1);
    }
    // the smoothing row is read whatever ksm holds (q when there is none) so
    // the loads in flight stay countable; every wave rotates, wave 0 stores
    float fac[QIT][8];
#pragma unroll
    for (int i = 0; i < QIT; ++i) {
      const float4* fp = reinterpret_cast<const float4*>(
          ksm != nullptr ? ksm + (((int64_t)b * Hkv + kv) % ksm_rows) * D + (lane % L) * 8
                         : q + (lane % L) * 8);
      const float4 f0 = fp[0], f1 = fp[1];
      fac[i][0] = f0.x; fac[i][1] = f0.y; fac[i][2] = f0.z; fac[i][3] = f0.w;
      fac[i][4] = f1.x; fac[i][5] = f1.y; fac[i][6] = f1.z; fac[i][7] = f1.w;
    }
    // the code rows go out after the query, codebook and factor loads:
    // loads complete in order, so the rotation and the table wait for
    // those alone while the rows stream in
    prefetch_rows(kcodes, cpre);
    prefetch_rows(vcodes, vpre);
#pragma unroll
    for (int i = 0; i < QIT; ++i) {
      const int r = i * QROWS + lane / L;
      float v[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = ksm != nullptr ? qraw[i][e] * fac[i][e] : qraw[i][e];
      hadamard_row<8, L>(v, lane);
      const float rs = scale * rsqrt_pow2(D);
      if (wave == 0 && r < RP) {
#pragma unroll
        for (int e = 0; e < 8; ++e) qs[r][(lane % L) * 8 + e] = v[e] * rs;
      }
    }
    __syncthreads();
    if (fast) {
      const int gsub = tid / 32, cl = tid % 32;
      auto half_entries = [&](const float4 (&cb)[4][2], int sg, int half, const float (&qv)[RP][8]) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float cv[8] = {cb[i][0].x, cb[i][0].y, cb[i][0].z, cb[i][0].w,
                               cb[i][1].x, cb[i][1].y, cb[i][1].z, cb[i][1].w};
          float acc[RP];
#pragma unroll
          for (int r = 0; r < RP; ++r) {
            acc[r] = 0.0f;
#pragma unroll
            for (int j = 0; j < 8; ++j) acc[r] = __builtin_fmaf(qv[r][j], cv[j], acc[r]);
          }
          const int it = sg * 256 + cl + 32 * (half * 4 + i);
          if constexpr (RP == 4) {
            *reinterpret_cast<float4*>(tabf + it * 4) = make_float4(acc[0], acc[1], acc[2], acc[3]);
          } else if constexpr (RP == 2) {
            *reinterpret_cast<float2*>(tabf + it * 2) = make_float2(acc[0], acc[1]);
          } else {
            tabf[it] = acc[0];
          }
        }
      };
      for (int pass = 0; pass < npass; ++pass) {
        const int sg = 16 * pass + gsub;
        const bool own = sg < SG;
        const int g = (own ? sg : 0) % G;
        float qv[RP][8];
#pragma unroll
        for (int r = 0; r < RP; ++r) {
          const float4* qp = reinterpret_cast<const float4*>(&qs[r][g * 8]);
          const float4 x0 = qp[0], x1 = qp[1];
          qv[r][0] = x0.x; qv[r][1] = x0.y; qv[r][2] = x0.z; qv[r][3] = x0.w;
          qv[r][4] = x1.x; qv[r][5] = x1.y; qv[r][6] = x1.z; qv[r][7] = x1.w;
        }
        if (own) half_entries(cb0, sg, 0, qv);
        if (pass + 1 < npass) load_half(cb0, pass + 1, 0);
        if (own) half_entries(cb1, sg, 1, qv);
        if (pass + 1 < npass) load_half(cb1, pass + 1, 1);
      }
    } else {
      for (int it = tid; it < nit; it += CH_THREADS) {
        const int g = (it / C) % G;
        const float* cp = kcb + (int64_t)it * dsub;
        float acc[RP];
#pragma unroll
        for (int r = 0; r < RP; ++r) acc[r] = 0.0f;
        for (int j = 0; j < dsub; ++j) {
          const float c = cp[j];
#pragma unroll
          for (int r = 0; r < RP; ++r) acc[r] = __builtin_fmaf(qs[r][g * dsub + j], c, acc[r]);
        }
#pragma unroll
        for (int r = 0; r < RP; ++r) tabf[it * RP + r] = acc[r];
      }
    }
  } else {
    // ---- stage this unit's LUT: whole 1 KiB pieces straight into LDS, tail by hand
    const uint8_t* src = reinterpret_cast<const uint8_t*>(lut) +
                         ((size_t)b * Hkv * n_hsplit + unit) * lut_slice;
    const int bytes = tabn * 4;
    const int full = bytes / 1024;
    for (int piece = wave; piece < full; piece += CH_THREADS / 64)
      __builtin_amdgcn_global_load_lds(src + piece * 1024 + lane * 16,
                                       (__attribute__((address_space(3))) void*)(smem + piece * 1024),
                                       16, 0, 0);
    for (int i = full * 256 + tid; i < tabn; i += CH_THREADS)
      tabu[i] = reinterpret_cast<const uint32_t*>(src)[i];
    __builtin_amdgcn_s_waitcnt(0x0f70);                  // vmcnt(0)
  }
  // window slice rows: in flight during pass 1, used after it
  uint4 wkraw, wvraw;
  float wq[RP][8], wsc[RP];
  bool wact;
  {
    const int wa = ci * wslice < W ? ci * wslice : W;
    const int wb = (wa + wslice) < W ? (wa + wslice) : W;
    wact = win_slice_load<RP, D>(wkraw, wvraw, wq, q, kw, vw, wslice > 0, b, kv, h0, nh, Hq, Hkv,
                                 wstride, wa, wb, tid);
  }
  __syncthreads();

  float sc[CH_TPT][RP];
  // ---- pass 1: K scores (LUT gathers, RP heads per read)
#pragma unroll
  for (int k = 0; k < CH_TPT; ++k) {
    const int t = t0 + tid + CH_THREADS * k;
#pragma unroll
    for (int r = 0; r < RP; ++r) sc[k][r] = -__builtin_inff();
    if (t < t1) {
      float acc[RP];
#pragma unroll
      for (int r = 0; r < RP; ++r) acc[r] = 0.0f;
      auto gather = [&](int sg, int z) { lut_add<RP>(tabf, (sg * C + z) * RP, acc); };
      if constexpr (SGC != 0) {
        uint4 w[SGW];
        if (k < KP) {
#pragma unroll
          for (int i = 0; i < SGW; ++i) w[i] = cpre[k < KP ? k : 0][i];
        } else {
          load_codes<SGC>(kcodes + (rowbase + t) * SG, w);
        }
        visit_codes<SGC>(w, C, gather);
      } else {
        for_codes<SGC>(kcodes + (rowbase + t) * SG, SG, C, gather);
      }
#pragma unroll
      for (int r = 0; r < RP; ++r) sc[k][r] = acc[r];
    }
  }
  if (wslice > 0) win_slice_scores<RP, D>(wsc, wkraw, wq, wact, scale);
  if constexpr (!FUSE) prefetch_rows(vcodes, vpre);   // after the window row's wait
  // ---- chunk max per head
#pragma unroll
  for (int r = 0; r < RP; ++r) {
    float v = -__builtin_inff();
#pragma unroll
    for (int k = 0; k < CH_TPT; ++k) v = fmaxf(v, sc[k][r]);
    v = wave_max(v);
    if (lane == 0) red_f[wave][r] = v;
    if (wslice > 0) {
      const float vw = wave_max(wsc[r]);
      if (lane == 0) red_wf[wave][r] = vw;
    }
  }
  __syncthreads();                                      // also: every LUT read is done
  // chunk max per head (every thread folds the wave maxima itself), then the
  // weights p = exp(s - m) in place of the scores and their per-head sum
  float m[RP];
#pragma unroll
  for (int r = 0; r < RP; ++r) {
    float v = red_f[0][r];
    for (int w = 1; w < CH_THREADS / 64; ++w) v = fmaxf(v, red_f[w][r]);
    m[r] = v;
  }
  if (tid < RP) {
    float v = red_f[0][tid], vw = red_wf[0][tid];
    for (int w = 1; w < CH_THREADS / 64; ++w) {
      v = fmaxf(v, red_f[w][tid]);
      vw = fmaxf(vw, red_wf[w][tid]);
    }
    mx[tid] = v;
    mxw[tid] = vw;
  }
#pragma unroll
  for (int r = 0; r < RP; ++r) {
    float sp = 0.0f;
#pragma unroll
    for (int k = 0; k < CH_TPT; ++k) {
      sc[k][r] = __expf(sc[k][r] - m[r]);               // -inf (no token) -> 0
      sp += sc[k][r];
    }
    sp = wave_sum(sp);
    if (lane == 0) red_l[wave][r] = sp;
  }
  for (int i = tid; i < tabh / 4; i += CH_THREADS)
    reinterpret_cast<uint4*>(tabu)[i] = make_uint4(0u, 0u, 0u, 0u);
  for (int i = (tabh / 4) * 4 + tid; i < tabh; i += CH_THREADS) tabu[i] = 0u;
  __syncthreads();
  // fraction bits per head from the chunk's own weight sum l (>= 1, the
  // maximum's weight): F = 31 - ceil(log2 l) keeps l * 2^F <= 2^31, so every
  // bin, every 32-bit field and the integer sum of the chunk stay below 2^32,
  // while a weight dropped by rounding is below 2^-F-1 <= l * 2^-32: the
  // mass lost to rounding is at most chunk * 2^-32 of l however peaky the
  // chunk.
  float fsc[RP], finv[RP];
#pragma unroll
  for (int r = 0; r < RP; ++r) {
    float l = red_l[0][r];
    for (int w = 1; w < CH_THREADS / 64; ++w) l += red_l[w][r];
    const int F = 31 - ceil_log2_f(l);
    fsc[r] = (float)(1u << F);
    finv[r] = 1.0f / fsc[r];
  }
  uint32_t ls[RP];
#pragma unroll
  for (int r = 0; r < RP; ++r) ls[r] = 0u;

  // ---- window slice: p = exp(s - m_w), p * H v / sqrt(D) summed over the
  // rows of each wave into LDS slot [wave][r][D] (the contraction's region,
  // free until pass 2 ends), sum p over the rows into red_wl
  if (wslice > 0) {
    const uint32_t vr[4] = {wvraw.x, wvraw.y, wvraw.z, wvraw.w};
    float vx[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      vx[2 * i] = f16_bits_to_f32(vr[i]);
      vx[2 * i + 1] = f16_bits_to_f32(vr[i] >> 16);
    }
    hadamard_row<8, L>(vx, lane);
    constexpr float rs = rsqrt_pow2(D);
#pragma unroll
    for (int e = 0; e < 8; ++e) vx[e] *= rs;
    const int col = tid % L;
#pragma unroll
    for (int r = 0; r < RP; ++r) {
      const float pf = wact ? __expf(wsc[r] - mxw[r]) : 0.0f;
      const float lw = wave_sum(col == 0 ? pf : 0.0f);
      if (lane == 0) red_wl[wave][r] = lw;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float a = pf * vx[e];
        if constexpr (L <= 8) a += xor_lane<8>(a);    // rows of the wave: lanes L .. 32 apart
        if constexpr (L <= 16) a = pair_sum<16>(a);
        a = pair_sum<32>(a);
        if (lane < L) cpart[(wave * RP + r) * D + col * 8 + e] = a;
      }
    }
  }

  // ---- pass 2: fixed-point weights into the V histogram
#pragma unroll
  for (int k = 0; k < CH_TPT; ++k) {
    const int t = t0 + tid + CH_THREADS * k;
    if (t < t1) {
      uint32_t pw[RP];
#pragma unroll
      for (int r = 0; r < RP; ++r) {
        pw[r] = (uint32_t)__builtin_rintf(sc[k][r] * fsc[r]);
        ls[r] += pw[r];
      }
      auto scatter = [&](int sg, int z) { hist_add<RP>(tabu, sg, z, C, pw); };
      if constexpr (SGC != 0) {
        uint4 w[SGW];
        if (k < KP) {
#pragma unroll
          for (int i = 0; i < SGW; ++i) w[i] = vpre[k < KP ? k : 0][i];
        } else {
          load_codes<SGC>(vcodes + (rowbase + t) * SG, w);
        }
        visit_codes<SGC>(w, C, scatter);
      } else {
        for_codes<SGC>(vcodes + (rowbase + t) * SG, SG, C, scatter);
      }
    }
  }
#pragma unroll
  for (int r = 0; r < RP; ++r) {
    const uint32_t v = wave_sum_u32(ls[r]);
    if (lane == 0) red_u[wave][r] = v;
  }
  __syncthreads();
  if (tid < RP) {
    uint32_t v = 0u;
    float vw = 0.0f;
    for (int w = 0; w < CH_THREADS / 64; ++w) {
      v += red_u[w][tid];
      vw += red_wl[w][tid];
    }
    lt[tid] = v;
    ltw[tid] = vw;
  }
  constexpr int NO = (RP * D + CH_THREADS - 1) / CH_THREADS;   // outputs per thread
  float wsum[NO];
#pragma unroll
  for (int j = 0; j < NO; ++j) wsum[j] = 0.0f;
  if (wslice > 0) {                                     // window rows, summed over waves
#pragma unroll
    for (int j = 0; j < NO; ++j) {
      const int o = tid + CH_THREADS * j;
      if (o < RP * D)
        for (int w = 0; w < CH_THREADS / 64; ++w) wsum[j] += cpart[w * RP * D + o];
    }
    __syncthreads();                                    // before the contraction reuses it
  }

  // ---- o_rot[r][g*dsub + j] = 2^-F sum_s sum_c W[s][g][c][r] * C^V_sg[c][j].
  // Item (s, codeword part, 4 consecutive dims): float4 codebook loads,
  // histogram entries broadcast to the lanes sharing a codeword.  Groups of
  // 2 dims (4-bit scalar codes through their product codebook) take items of
  // one group each, with float2 loads.
  const int dsub = D / G;
  constexpr int D4 = D / 4;
  const int P = cparts;
  const int cper = (C + P - 1) / P;
  if (dsub == 2) {
    constexpr int D2 = D / 2;
    for (int it = tid; it < S * P * D2; it += CH_THREADS) {
      const int g = it % D2;
      const int rest = it / D2;
      const int pi = rest % P, s = rest / P;
      const int sg = s * G + g;
      const int c0 = pi * cper, c1 = (c0 + cper) < C ? (c0 + cper) : C;
      float acc[RP][2];
#pragma unroll
      for (int r = 0; r < RP; ++r) acc[r][0] = acc[r][1] = 0.0f;
      const float* cvp = vcb + (int64_t)sg * C * 2;
      const uint32_t* hp = tabu + sg * hist_stride(C, RP);
#pragma unroll 16
      for (int c = c0; c < c1; ++c) {
        const float2 cv = *reinterpret_cast<const float2*>(cvp + (int64_t)c * 2);
#pragma unroll
        for (int r = 0; r < RP; ++r) {
          const float w = (float)hp[hist_bin<RP>(c, r, C)];
          acc[r][0] = __builtin_fmaf(w, cv.x, acc[r][0]);
          acc[r][1] = __builtin_fmaf(w, cv.y, acc[r][1]);
        }
      }
#pragma unroll
      for (int r = 0; r < RP; ++r)
        *reinterpret_cast<float2*>(cpart + ((s * P + pi) * RP + r) * D + 2 * g) =
            make_float2(acc[r][0], acc[r][1]);
    }
  }
  for (int it = tid; dsub >= 4 && it < S * P * D4; it += CH_THREADS) {
    const int d4 = it % D4;
    const int rest = it / D4;
    const int pi = rest % P, s = rest / P;
    const int d0 = d4 * 4;
    const int g = d0 / dsub, j0 = d0 - g * dsub;
    const int sg = s * G + g;
    const int c0 = pi * cper, c1 = (c0 + cper) < C ? (c0 + cper) : C;
    float acc[RP][4];
#pragma unroll
    for (int r = 0; r < RP; ++r)
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[r][e] = 0.0f;
    const float* cvp = vcb + (int64_t)sg * C * dsub + j0;
    const uint32_t* hp = tabu + sg * hist_stride(C, RP);
#pragma unroll 16
    for (int c = c0; c < c1; ++c) {
      const float4 cv = *reinterpret_cast<const float4*>(cvp + (int64_t)c * dsub);
#pragma unroll
      for (int r = 0; r < RP; ++r) {
        const float w = (float)hp[hist_bin<RP>(c, r, C)];
        acc[r][0] = __builtin_fmaf(w, cv.x, acc[r][0]);
        acc[r][1] = __builtin_fmaf(w, cv.y, acc[r][1]);
        acc[r][2] = __builtin_fmaf(w, cv.z, acc[r][2]);
        acc[r][3] = __builtin_fmaf(w, cv.w, acc[r][3]);
      }
    }
#pragma unroll
    for (int r = 0; r < RP; ++r)
      *reinterpret_cast<float4*>(cpart + ((s * P + pi) * RP + r) * D + d0) =
          make_float4(acc[r][0], acc[r][1], acc[r][2], acc[r][3]);
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < NO; ++j) {
    const int o = tid + CH_THREADS * j;
    const int r = o / D, d = o - r * D;
    if (o >= RP * D || r >= nh) continue;
    float inv = finv[0];
#pragma unroll
    for (int rr = 1; rr < RP; ++rr) inv = r == rr ? finv[rr] : inv;
    float v = 0.0f;
    for (int sp = 0; sp < S * P; ++sp) v += cpart[(sp * RP + r) * D + d];
    v *= inv;
    float m = mx[r], l = (float)lt[r] * inv;
    if (wslice > 0) {                                   // fold the window slice in
      const float mw = mxw[r];
      const float mm = fmaxf(m, mw);
      const float a = __expf(m - mm);
      const float aw = mw == -__builtin_inff() ? 0.0f : __expf(mw - mm);
      v = v * a + wsum[j] * aw;
      l = l * a + ltw[r] * aw;
      m = mm;
    }
    float* pp = part + ((int64_t)(b * Hq + h0 + r) * nslots + ci) * pstride;
    pp[4 + d] = v;
    if (d == 0) { pp[0] = m; pp[1] = l; }
  }
}

// ------------------------------------------------------------- attn_merge
// grid (B*Hq), block 256.  Every record holds a softmax partial (m, l, o)
// with o in the rotated domain (coded chunks, window slices folded in, window
// blocks).  out = H (sum_i w_i o_i) / (sqrt(D) sum_i w_i l_i) with
// w_i = exp(m_i - max_j m_j); the two block halves take alternate records.
template <int D>
__global__ __launch_bounds__(256) void attn_merge_kernel(const float* __restrict__ part,
                                                         float* __restrict__ out, int nslots,
                                                         int pstride) {
  constexpr int L = D / 8;
  __shared__ float crot[2][D];
  __shared__ float wts[256];
  __shared__ float red[8];
  const int bh = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane % L;
  const float* pb = part + (int64_t)bh * nslots * pstride;
  float mloc = -__builtin_inff();
  for (int i = tid; i < nslots; i += 256) mloc = fmaxf(mloc, pb[(int64_t)i * pstride]);
  mloc = wave_max(mloc);
  if (lane == 0) red[wave] = mloc;
  __syncthreads();
  const float ms = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  float den = 0.0f;
  const int half = tid >> 7, d = tid & 127;
  float o0 = 0.0f, o1 = 0.0f;                           // dims d and d + 128
  for (int i0 = 0; i0 < nslots; i0 += 256) {
    const int i = i0 + tid;
    float wgt = 0.0f, lv = 0.0f;
    if (i < nslots) {
      const float mi = pb[(int64_t)i * pstride];
      wgt = mi == -__builtin_inff() ? 0.0f : __expf(mi - ms);
      lv = pb[(int64_t)i * pstride + 1];
    }
    wts[tid] = wgt;
    den += wgt * lv;
    __syncthreads();
    const int n = (nslots - i0) < 256 ? (nslots - i0) : 256;
    if (d < D) {
#pragma unroll 8
      for (int k = half; k < n; k += 2) {
        const float* rec = pb + (int64_t)(i0 + k) * pstride + 4;
        o0 = __builtin_fmaf(wts[k], rec[d], o0);
        if (D > 128) o1 = __builtin_fmaf(wts[k], rec[d + 128], o1);
      }
    }
    __syncthreads();
  }
  den = wave_sum(den);
  if (lane == 0) red[4 + wave] = den;
  if (d < D) crot[half][d] = o0;
  if (D > 128) crot[half][d + 128] = o1;
  __syncthreads();
  const float total = red[4] + red[5] + red[6] + red[7];
  if (tid < 64) {                                        // one wave unrotates
    float v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = crot[0][col * 8 + e] + crot[1][col * 8 + e];
    hadamard_row<8, L>(v, lane);
    if (lane < L) {
      constexpr float sc = rsqrt_pow2(D);
      const float inv = sc / total;
      float4* op = reinterpret_cast<float4*>(out + (int64_t)bh * D + col * 8);
      op[0] = make_float4(v[0] * inv, v[1] * inv, v[2] * inv, v[3] * inv);
      op[1] = make_float4(v[4] * inv, v[5] * inv, v[6] * inv, v[7] * inv);
    }
  }
}

// --------------------------------------------------------------- launcher
template <int RP>
static hipError_t launch_rp(const AttnPlan& p, int SG, const float* q, const float* kcb,
                            const uint8_t* kc, const uint8_t* vc, const float* vcb, float* lut,
                            float* part, const uint16_t* kw, const uint16_t* vw, int B, int Hq,
                            int Hkv, int D, int S, int G, int C, int Tc, int W, int cstride,
                            int wstride, float scale, Smooth ksm, hipStream_t st) {
  hipError_t e = hipSuccess;
  size_t lds = 0;
  if (p.n_chunks > 0 && !p.fuse_lut) {
    if (D == 64)
      attn_lut_kernel<RP, 64><<<dim3(B * Hkv * p.n_hsplit, SG), 256, 0, st>>>(
          q, kcb, lut, Hq, Hkv, p.n_hsplit, G, C, p.lut_slice, scale, ksm.f, ksm.n_scale);
    else if (D == 128)
      attn_lut_kernel<RP, 128><<<dim3(B * Hkv * p.n_hsplit, SG), 256, 0, st>>>(
          q, kcb, lut, Hq, Hkv, p.n_hsplit, G, C, p.lut_slice, scale, ksm.f, ksm.n_scale);
    else
      attn_lut_kernel<RP, 256><<<dim3(B * Hkv * p.n_hsplit, SG), 256, 0, st>>>(
          q, kcb, lut, Hq, Hkv, p.n_hsplit, G, C, p.lut_slice, scale, ksm.f, ksm.n_scale);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (p.n_chunks > 0) {
    const size_t tab = (((size_t)SG * hist_stride(C, RP) * 4) + 15) & ~(size_t)15;
    lds = tab + (size_t)S * p.cparts * RP * D * 4;
  }
  if (p.n_wblocks > 0) {
    const size_t wl = ((size_t)ATTN_WIN_BLOCK * RP + (size_t)8 * RP * D) * 4;
    if (wl > lds) lds = wl;
  }
  if (p.wslice > 0 && S * p.cparts < 8)               // window row sums need 8 slots
    lds = ((((size_t)SG * hist_stride(C, RP) * 4) + 15) & ~(size_t)15) + (size_t)8 * RP * D * 4;
  dim3 grid(p.n_chunks + p.n_wblocks, Hkv * p.n_hsplit, B);
  const int nslots = p.n_chunks + p.n_wblocks;
#define KVQ_CH(SGV, DV)                                                                        \
  {                                                                                            \
    auto kern = p.fuse_lut ? attn_chunk_kernel<RP, SGV, DV, true>                              \
                           : attn_chunk_kernel<RP, SGV, DV, false>;                            \
    e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize,     \
                            (int)lds);                                                         \
    if (e != hipSuccess) return e;                                                             \
    kern<<<grid, CH_THREADS, lds, st>>>(kc, vc, vcb, lut, part, Hq, Hkv, S, G, C, Tc,          \
                                        p.n_chunks, p.chunk, p.n_hsplit, p.pstride,            \
                                        p.cparts, p.lut_slice, kcb, q, kw, vw, W,              \
                                        p.wslice, nslots, scale, cstride, wstride, ksm.f,      \
                                        ksm.n_scale);                                          \
    return hipGetLastError();                                                                  \
  }
  if (D == 64) KVQ_CH(0, 64)
  if (D == 256) KVQ_CH(0, 256)
  if (SG == 16) KVQ_CH(16, 128)
  if (SG == 32) KVQ_CH(32, 128)
  if (SG == 64) KVQ_CH(64, 128)
  KVQ_CH(0, 128)
#undef KVQ_CH
}

hipError_t launch_attend(const AttnPlan& p, int B, int Hq, int Hkv, int D, int S, int G, int C,
                         int Tc, int W, int cstride, int wstride, float scale, const float* q,
                         const uint8_t* kc,
                         const uint8_t* vc, const float* kcb, const float* vcb,
                         const uint16_t* kw, const uint16_t* vw, float* out, void* ws,
                         Smooth ksm, hipStream_t st) {
  float* lut = reinterpret_cast<float*>(ws);
  float* part = reinterpret_cast<float*>(reinterpret_cast<uint8_t*>(ws) +
                                         ((p.lut_bytes + 255) & ~(size_t)255));
  const int SG = S * G;
  hipError_t e;
  if (p.rc) e = launch_attend_rc(p, B, Hq, Hkv, S, G, Tc, W, cstride, wstride, scale, q, kc, vc, kcb,
                                 vcb, kw, vw, reinterpret_cast<uint8_t*>(lut), part, ksm, st);
  else if (p.rp == 4) e = launch_rp<4>(p, SG, q, kcb, kc, vc, vcb, lut, part, kw, vw, B, Hq, Hkv, D, S, G, C, Tc, W, cstride, wstride, scale, ksm, st);
  else if (p.rp == 2) e = launch_rp<2>(p, SG, q, kcb, kc, vc, vcb, lut, part, kw, vw, B, Hq, Hkv, D, S, G, C, Tc, W, cstride, wstride, scale, ksm, st);
  else e = launch_rp<1>(p, SG, q, kcb, kc, vc, vcb, lut, part, kw, vw, B, Hq, Hkv, D, S, G, C, Tc, W, cstride, wstride, scale, ksm, st);
  if (e != hipSuccess) return e;
  const int nslots = p.n_chunks + p.n_wblocks;
  if (D == 64) attn_merge_kernel<64><<<dim3(B * Hq), 256, 0, st>>>(part, out, nslots, p.pstride);
  else if (D == 128) attn_merge_kernel<128><<<dim3(B * Hq), 256, 0, st>>>(part, out, nslots, p.pstride);
  else attn_merge_kernel<256><<<dim3(B * Hq), 256, 0, st>>>(part, out, nslots, p.pstride);
  return hipGetLastError();
}

}  // namespace kvq
