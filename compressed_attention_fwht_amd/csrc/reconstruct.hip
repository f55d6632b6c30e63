// K3 -- reconstruction from codes: x_rot[g*dsub + j] = sum_s C_sg[z_sg][j],
// optionally followed by the inverse rotation x = H_D x_rot.
//
// "VQKV" summary, 2. Methodology (RSimVQ reconstruction as the sum of the
// retrieved entries); "VeloxQuant-MLX 0.5.1", Architecture (decode by summing
// stage outputs, then unrotate).
//
// The stage sum is accumulated in float64 and rounded once to float32, so the
// result is the correctly rounded sum whatever the stage order.  HBM-bound by
// the 4*D-byte float32 output per vector.
//
// Lane layout: L = D/8 lanes per row; lane c of a row holds the dims
// [4c, 4c+4) (elements 0..3) and [D/2 + 4c, D/2 + 4c + 4) (elements 4..7).
// Each of the two 16-byte stores of a lane then lands next to its
// neighbours' (a row's lanes write two contiguous D*2-byte halves).  The
// layout is a permutation of the bits of the dim index (the top bit becomes
// the element's bit 2), and the Walsh-Hadamard matrix is unchanged by
// permuting the index bits of rows and columns alike, so the butterfly over
// (lane, element) computes the same transform.
//
// Three variants.  With 2 to 4 stages whose first two stages' codebooks for
// half the dims fit in LDS (2*C*D/2*4 bytes up to RC_LDS_MAX), the half-table
// kernel holds each half's tables of those stages in LDS in turn (later
// stages are gathered through the caches).  Otherwise,
// with 1, 2 or 4 stages (4 only below D = 256) whose per-stage codebooks fit
// in LDS (G*C*dsub*4 bytes up to RC_LDS_MAX), each block copies its book's
// stage-0 codebooks into LDS once (and its code rows too, when they fit
// beside them) and codes a range of that book's vectors: the stage-0 gathers
// are LDS reads, later stages' go through the caches.  Otherwise every gather
// goes through the caches (a grid-stride loop over all vectors).
#include "kvq_internal.h"
#include <type_traits>

namespace kvq {

constexpr int RC_THREADS = 512;              // cache variant
constexpr int RC_LDS_THREADS = 1024;         // LDS variant: one block per CU at 128 KiB
constexpr int RC_UNR = 2;                    // vectors per lane per iteration
constexpr size_t RC_LDS_MAX = 128 * 1024;    // stage-0 codebooks in LDS, at most
constexpr size_t RC_LDS_BLOCK = 160 * 1024;  // LDS of one CU

// Code bytes of RC_UNR vectors for a lane: stages s < SS, groups ga and gb.
template <int SS>
struct RcCodes {
  int za[RC_UNR][SS], zb[RC_UNR][SS];
};

// Finish RC_UNR vectors of a lane (their float32 sums): optional unrotation
// and smoothing, the two 16-byte stores.
template <int D>
__device__ __forceinline__ void rc_finish(float (&sum)[RC_UNR][8], float* __restrict__ out,
                                          const int64_t (&vec)[RC_UNR],
                                          const bool (&live)[RC_UNR], int64_t n_per_book,
                                          int unrotate, const float* __restrict__ smooth,
                                          int64_t n_scale, int64_t n_rows, int lane, int da,
                                          int db) {
  constexpr int L = D / 8;
#pragma unroll
  for (int u = 0; u < RC_UNR; ++u) {
    float v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = sum[u][e];
    if (unrotate) {                         // uniform branch: all lanes take it
      hadamard_row<8, L>(v, lane);
      constexpr float sc = rsqrt_pow2(D);
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] *= sc;
    }
    if (smooth != nullptr && live[u]) {     // dual transform undone: times the factors
      const int64_t book = vec[u] / n_per_book;
      const int64_t seq = (vec[u] - book * n_per_book) / n_rows;
      const float* lp = smooth + (book * n_scale + seq % n_scale) * D;
      const float4 a = *reinterpret_cast<const float4*>(lp + da);
      const float4 b = *reinterpret_cast<const float4*>(lp + db);
      v[0] *= a.x; v[1] *= a.y; v[2] *= a.z; v[3] *= a.w;
      v[4] *= b.x; v[5] *= b.y; v[6] *= b.z; v[7] *= b.w;
    }
    if (live[u]) {
      float* o = out + vec[u] * D;
      *reinterpret_cast<float4*>(o + da) = make_float4(v[0], v[1], v[2], v[3]);
      *reinterpret_cast<float4*>(o + db) = make_float4(v[4], v[5], v[6], v[7]);
    }
  }
}

// LDS variant (SS = S stages: 1, 2 or 4; stage 0 in LDS): grid (blocks per
// book, n_books);
// block (x, book) copies the book's stage-0 codebooks into LDS and codes its vectors
// [x*per, (x+1)*per).  PRE: the block's code rows are copied into LDS beside
// the codebooks up front, so the stream that follows only writes to HBM
// (reads between the writes cost measurable bandwidth); otherwise the code
// bytes of a wave's next RC_UNR x ROWS vectors are loaded while the current
// ones are summed and stored.
template <int D, int SS, bool PRE>
__global__ __launch_bounds__(RC_LDS_THREADS) void reconstruct_lds_kernel(
    const uint8_t* __restrict__ codes, const float* __restrict__ cb, float* __restrict__ out,
    int64_t n_per_book, int64_t per_block, int G, int C, int dsub, int unrotate,
    const float* __restrict__ smooth, int64_t n_scale, int64_t n_rows) {
  constexpr int L = D / 8;
  constexpr int ROWS = 64 / L;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const float* cbl = reinterpret_cast<const float*>(smem);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane % L;
  const int da = 4 * col, db = D / 2 + 4 * col;
  const int ga = da / dsub, ja = da - ga * dsub;
  const int gb = db / dsub, jb = db - gb * dsub;
  const int64_t book = blockIdx.y;
  const int64_t book_stride = (int64_t)SS * G * C * dsub;
  const int64_t stage_stride = (int64_t)G * C * dsub;
  const float* cbg = cb + book * book_stride;
  const int64_t v0 = (int64_t)blockIdx.x * per_block;
  const int64_t v1 = (v0 + per_block) < n_per_book ? (v0 + per_block) : n_per_book;
  const int64_t first = book * n_per_book;              // global index of the book's vector 0
  constexpr int64_t STEP = (int64_t)ROWS * (RC_LDS_THREADS / 64);
  auto rows_of = [&](int64_t wbase, int64_t (&vec)[RC_UNR], bool (&live)[RC_UNR]) {
#pragma unroll
    for (int u = 0; u < RC_UNR; ++u) {
      const int64_t v = wbase + lane / L + u * STEP;
      live[u] = v < v1;
      vec[u] = first + (live[u] ? v : v1 - 1);
    }
  };
  // PRE: the code rows sit in LDS after the codebooks at the same offset
  // modulo 16 as in global memory (whole 16-byte pieces copied as such, the
  // partial first and last pieces byte by byte)
  const int SG = SS * G;
  uint8_t* lcodes = smem + stage_stride * 4;
  const int64_t a0 = (first + v0) * SG;
  const int lo = (int)(a0 & 15);
  auto code_row = [&](int64_t v) -> const uint8_t* {    // v: global vector index
    if constexpr (PRE) return lcodes + lo + (v - first - v0) * SG;
    else return codes + v * SG;
  };
  auto load_codes_of = [&](RcCodes<SS>& k, const int64_t (&vv)[RC_UNR]) {
#pragma unroll
    for (int u = 0; u < RC_UNR; ++u)
#pragma unroll
      for (int s = 0; s < SS; ++s) {
        const uint8_t* row = code_row(vv[u]) + s * G;
        k.za[u][s] = row[ga];
        k.zb[u][s] = row[gb];
      }
  };
  int64_t wbase = v0 + wave * ROWS;
  int64_t vec[RC_UNR];
  bool live[RC_UNR];
  rows_of(wbase, vec, live);
  RcCodes<SS> cur;
  if constexpr (!PRE) load_codes_of(cur, vec);          // in flight across the codebook copy
  const float4* src = reinterpret_cast<const float4*>(cbg);
  for (int64_t i = threadIdx.x; i < stage_stride / 4; i += RC_LDS_THREADS)
    reinterpret_cast<float4*>(smem)[i] = src[i];
  if constexpr (PRE) {
    const int64_t nbytes = (v1 - v0) * SG;
    const int64_t nchunk = (lo + nbytes + 15) / 16;
    for (int64_t i = threadIdx.x; i < nchunk; i += RC_LDS_THREADS) {
      const int64_t g0 = a0 - lo + 16 * i;
      if (g0 >= a0 && g0 + 16 <= a0 + nbytes) {
        reinterpret_cast<uint4*>(lcodes)[i] = *reinterpret_cast<const uint4*>(codes + g0);
      } else {
        for (int b = 0; b < 16; ++b)
          if (g0 + b >= a0 && g0 + b < a0 + nbytes) lcodes[16 * i + b] = codes[g0 + b];
      }
    }
  }
  __syncthreads();
  if constexpr (PRE) load_codes_of(cur, vec);
  // the loop bound is wave-uniform: every lane joins the butterfly
  for (; wbase < v1; wbase += STEP * RC_UNR) {
    int64_t nvec[RC_UNR];
    bool nlive[RC_UNR];
    rows_of(wbase + STEP * RC_UNR, nvec, nlive);
    RcCodes<SS> nxt;
    load_codes_of(nxt, nvec);
    // one or two stages: the float32 sum is already the correctly rounded
    // one (a single entry, or one rounding of the sum of two floats); four:
    // float64, rounded once
    using Acc = typename std::conditional<(SS <= 2), float, double>::type;
    Acc acc[RC_UNR][8];
#pragma unroll
    for (int u = 0; u < RC_UNR; ++u) {
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[u][e] = 0;
#pragma unroll
      for (int s = 0; s < SS; ++s) {
        const int za = cur.za[u][s] < C ? cur.za[u][s] : C - 1;
        const int zb = cur.zb[u][s] < C ? cur.zb[u][s] : C - 1;
        const float* base = s == 0 ? cbl : cbg + s * stage_stride;
        const float4 a = *reinterpret_cast<const float4*>(base + ((int64_t)ga * C + za) * dsub + ja);
        const float4 b = *reinterpret_cast<const float4*>(base + ((int64_t)gb * C + zb) * dsub + jb);
        acc[u][0] += a.x; acc[u][1] += a.y; acc[u][2] += a.z; acc[u][3] += a.w;
        acc[u][4] += b.x; acc[u][5] += b.y; acc[u][6] += b.z; acc[u][7] += b.w;
      }
    }
    float sum[RC_UNR][8];
#pragma unroll
    for (int u = 0; u < RC_UNR; ++u)
#pragma unroll
      for (int e = 0; e < 8; ++e) sum[u][e] = (float)acc[u][e];
    rc_finish<D>(sum, out, vec, live, n_per_book, unrotate, smooth, n_scale, n_rows, lane, da,
                 db);
    cur = nxt;
#pragma unroll
    for (int u = 0; u < RC_UNR; ++u) {
      vec[u] = nvec[u];
      live[u] = nlive[u];
    }
  }
}

// Half-table variant (2 to 4 stages; the first SL = 2 stages' tables for half
// the dims fit in LDS, later stages are gathered through the caches in the
// same ascending order): lane c of a row holds dims [4c, 4c+4) of the first half and
// [D/2 + 4c, D/2 + 4c + 4) of the second, and the groups of each half are
// contiguous in every stage's codebook.  A batch of RC_HK vectors per lane
// is coded in two phases: the block stages every stage's codebooks of one
// half's groups into LDS (SL*C*D/2 floats), every lane sums its dims of that
// half over the stages and keeps the 4 sums per vector in registers; then the
// other half's tables replace them and each vector is finished (unrotation,
// smoothing, stores) as soon as its second half is summed.  Consecutive
// batches take the halves in opposite orders, so a batch after the first
// loads one table, not two.  The batch's code rows are copied into LDS
// behind the table first, so every gather, of codes and of entries, is an
// LDS read.
// grid (blocks per book, n_books); block (x, book) codes its book's vectors
// [x*per, (x+1)*per).
constexpr int RC_HT_THREADS = 1024;
constexpr int RC_HK = 4;                     // vectors per lane per batch (8 spills)

template <int D, int S, int SL>
__global__ __launch_bounds__(RC_HT_THREADS) void reconstruct_half_kernel(
    const uint8_t* __restrict__ codes, const float* __restrict__ cb, float* __restrict__ out,
    int64_t n_per_book, int64_t per_block, int G, int C, int unrotate,
    const float* __restrict__ smooth, int64_t n_scale, int64_t n_rows) {
  static_assert(RC_HK % RC_UNR == 0, "vectors are finished RC_UNR at a time");
  constexpr int L = D / 8;
  constexpr int RPASS = RC_HT_THREADS / L;              // rows of one pass of the block
  constexpr int BATCH = RPASS * RC_HK;
  using Acc = typename std::conditional<(S <= 2), float, double>::type;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  float* tab = reinterpret_cast<float*>(smem);
  const int lane = threadIdx.x & 63;
  const int col = lane % L;
  const int rloc = threadIdx.x / L;                     // row within a pass
  const int dsub = D / G;
  const int GH = G / 2;                                 // groups per half
  const int da = 4 * col, db = D / 2 + 4 * col;
  const int64_t book = blockIdx.y;
  const int SG = S * G;
  const float* cbb = cb + book * (int64_t)S * G * C * dsub;
  const int64_t v0 = (int64_t)blockIdx.x * per_block;
  const int64_t v1 = (v0 + per_block) < n_per_book ? (v0 + per_block) : n_per_book;
  const int64_t first = book * n_per_book;
  const int64_t half_floats = (int64_t)GH * C * dsub;   // one stage of one half
  // code rows of the batch, behind the table, at the same offset modulo 16
  // as in global memory
  uint8_t* lcodes = smem + (size_t)SL * half_floats * 4;
  int loaded = -1;                                      // half held in LDS (block-uniform)
  int lo = 0;                                           // offset of the batch's first code byte

  // the code rows of vectors [vb, min(vb + BATCH, v1)) into lcodes + lo
  // (whole 16-byte pieces as such, the partial first and last bytewise);
  // block-uniform call, after a barrier that ends every read of the old rows
  auto load_codes = [&](int64_t vb) {
    const int64_t a0 = (first + vb) * SG;
    const int64_t vend = (vb + BATCH) < v1 ? (vb + BATCH) : v1;
    const int64_t nbytes = (vend - vb) * SG;
    lo = (int)(a0 & 15);
    const int64_t nchunk = (lo + nbytes + 15) / 16;
    for (int64_t i = threadIdx.x; i < nchunk; i += RC_HT_THREADS) {
      const int64_t g0 = a0 - lo + 16 * i;
      if (g0 >= a0 && g0 + 16 <= a0 + nbytes) {
        reinterpret_cast<uint4*>(lcodes)[i] = *reinterpret_cast<const uint4*>(codes + g0);
      } else {
        for (int b = 0; b < 16; ++b)
          if (g0 + b >= a0 && g0 + b < a0 + nbytes) lcodes[16 * i + b] = codes[g0 + b];
      }
    }
  };

  // one half's tables (and the batch's code rows when vb >= 0); block-uniform call
  auto load_half = [&](int hh, int64_t vb) {
    __syncthreads();                                    // every read of the old contents is done
    if (vb >= 0) load_codes(vb);
#pragma unroll
    for (int s = 0; s < SL; ++s) {
      const float4* src = reinterpret_cast<const float4*>(cbb + ((int64_t)s * G + hh * GH) * C * dsub);
      float4* dst = reinterpret_cast<float4*>(tab + s * half_floats);
      // four loads in flight per thread before their LDS stores (one at a
      // time, the reload measured 12 % of the kernel)
      const int64_t n4 = half_floats / 4;
      int64_t i = threadIdx.x;
      for (; i + 3 * RC_HT_THREADS < n4; i += 4 * RC_HT_THREADS) {
        float4 t[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) t[u] = src[i + u * RC_HT_THREADS];
#pragma unroll
        for (int u = 0; u < 4; ++u) dst[i + u * RC_HT_THREADS] = t[u];
      }
      for (; i < n4; i += RC_HT_THREADS) dst[i] = src[i];
    }
    __syncthreads();
    loaded = hh;
  };
  auto row_of = [&](int64_t vb, int k, int64_t& vec, bool& live) {
    const int64_t v = vb + (int64_t)k * RPASS + rloc;
    live = v < v1;
    vec = first + (live ? v : v1 - 1);
  };
  // this lane's 4 sums of half hh for vector vec of the batch at vb
  auto sum_half = [&](int hh, int64_t vb, int64_t vec, float (&r)[4]) {
    const int dh = hh ? db : da;
    const int g = dh / dsub, j = dh - g * dsub;
    const int gl = g - hh * GH;
    const uint8_t* row = lcodes + lo + (vec - first - vb) * SG + g;
    int z[S];
#pragma unroll
    for (int s = 0; s < S; ++s) {
      z[s] = row[s * G];
      z[s] = z[s] < C ? z[s] : C - 1;
    }
    Acc acc[4] = {0, 0, 0, 0};
#pragma unroll
    for (int s = 0; s < S; ++s) {                       // ascending stages
      const float4 e = s < SL
          ? *reinterpret_cast<const float4*>(tab + s * half_floats + ((int64_t)gl * C + z[s]) * dsub + j)
          : *reinterpret_cast<const float4*>(cbb + (((int64_t)s * G + g) * C + z[s]) * dsub + j);
      acc[0] += e.x; acc[1] += e.y; acc[2] += e.z; acc[3] += e.w;
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) r[e] = (float)acc[e];
  };
  // one batch: half h0 first, then half 1 - h0 with the finish
  auto batch = [&](int64_t vb, int h0) {
    if (loaded != h0) {
      load_half(h0, vb);
    } else {
      __syncthreads();                                  // every read of the old rows is done
      load_codes(vb);
      __syncthreads();
    }
    float hold[RC_HK][4];
#pragma unroll
    for (int k = 0; k < RC_HK; ++k) {
      int64_t vec;
      bool live;
      row_of(vb, k, vec, live);
      sum_half(h0, vb, vec, hold[k]);
      // one vector's LDS reads at a time: hoisting them all would spill
      __builtin_amdgcn_sched_barrier(0);
    }
    load_half(1 - h0, -1);
#pragma unroll
    for (int k = 0; k < RC_HK; k += RC_UNR) {
      int64_t vec[RC_UNR];
      bool live[RC_UNR];
      float sum[RC_UNR][8];
#pragma unroll
      for (int u = 0; u < RC_UNR; ++u) {
        row_of(vb, k + u, vec[u], live[u]);
        float r[4];
        sum_half(1 - h0, vb, vec[u], r);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          sum[u][e] = h0 == 0 ? hold[k + u][e] : r[e];
          sum[u][4 + e] = h0 == 0 ? r[e] : hold[k + u][e];
        }
      }
      rc_finish<D>(sum, out, vec, live, n_per_book, unrotate, smooth, n_scale, n_rows, lane, da,
                   db);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // the loop bounds are block-uniform: every thread takes part in the table
  // loads, barriers and butterflies
  for (int64_t vb = v0; vb < v1; vb += 2 * BATCH) {
    batch(vb, 0);
    if (vb + BATCH < v1) batch(vb + BATCH, 1);
  }
}

// Cache variant: grid-stride over every vector of every book, any S.
template <int D>
__global__ __launch_bounds__(RC_THREADS) void reconstruct_kernel(
    const uint8_t* __restrict__ codes, const float* __restrict__ cb, float* __restrict__ out,
    int64_t n_books, int64_t n_per_book, int G, int S, int C, int dsub, int unrotate,
    const float* __restrict__ smooth, int64_t n_scale, int64_t n_rows) {
  constexpr int L = D / 8;
  constexpr int ROWS = 64 / L;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane % L;
  const int da = 4 * col, db = D / 2 + 4 * col;
  const int ga = da / dsub, ja = da - ga * dsub;
  const int gb = db / dsub, jb = db - gb * dsub;
  const int SG = S * G;
  const int64_t n_total = n_books * n_per_book;
  const int64_t book_stride = (int64_t)S * G * C * dsub;
  const int64_t step = (int64_t)gridDim.x * (RC_THREADS / 64) * ROWS;
  // the loop bound is wave-uniform: every lane joins the butterfly
  for (int64_t wbase = ((int64_t)blockIdx.x * (RC_THREADS / 64) + wave) * ROWS; wbase < n_total;
       wbase += step * RC_UNR) {
    int64_t vec[RC_UNR];
    bool live[RC_UNR];
#pragma unroll
    for (int u = 0; u < RC_UNR; ++u) {
      const int64_t v = wbase + lane / L + u * step;
      live[u] = v < n_total;
      vec[u] = live[u] ? v : n_total - 1;
    }
    double acc[RC_UNR][8];
#pragma unroll
    for (int u = 0; u < RC_UNR; ++u)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[u][e] = 0.0;
    for (int s = 0; s < S; ++s) {
      int za[RC_UNR], zb[RC_UNR];
#pragma unroll
      for (int u = 0; u < RC_UNR; ++u) {
        const uint8_t* row = codes + vec[u] * SG + s * G;
        za[u] = row[ga];
        zb[u] = row[gb];
        za[u] = za[u] < C ? za[u] : C - 1;
        zb[u] = zb[u] < C ? zb[u] : C - 1;
      }
#pragma unroll
      for (int u = 0; u < RC_UNR; ++u) {
        const float* base = cb + (vec[u] / n_per_book) * book_stride;
        const float4 a = *reinterpret_cast<const float4*>(
            base + (((int64_t)s * G + ga) * C + za[u]) * dsub + ja);
        const float4 b = *reinterpret_cast<const float4*>(
            base + (((int64_t)s * G + gb) * C + zb[u]) * dsub + jb);
        acc[u][0] += a.x; acc[u][1] += a.y; acc[u][2] += a.z; acc[u][3] += a.w;
        acc[u][4] += b.x; acc[u][5] += b.y; acc[u][6] += b.z; acc[u][7] += b.w;
      }
    }
    float sum[RC_UNR][8];
#pragma unroll
    for (int u = 0; u < RC_UNR; ++u)
#pragma unroll
      for (int e = 0; e < 8; ++e) sum[u][e] = (float)acc[u][e];
    rc_finish<D>(sum, out, vec, live, n_per_book, unrotate, smooth, n_scale, n_rows, lane, da,
                 db);
  }
}

hipError_t launch_reconstruct(const uint8_t* codes, const float* cb, float* out, int64_t n_books,
                              int64_t n_per_book, int D, int G, int S, int C, int unrotate,
                              int64_t n_rows, Smooth sm, hipStream_t s) {
  const int64_t n = n_books * n_per_book;
  if (n == 0) return hipSuccess;
  const int dsub = D / G;
  const size_t cbytes = (size_t)G * C * dsub * sizeof(float);
  const int64_t vec_per_iter = (int64_t)(RC_THREADS / 64) * (64 / (D / 8)) * RC_UNR;
  // 2 to 4 stages whose first two stages' half-dim tables fit RC_LDS_MAX: the
  // half-table variant
  // (the LDS variants put the books on grid.y)
  const int SLc = S < 2 ? S : 2;                         // stages whose half tables sit in LDS
  const size_t hbytes = (size_t)SLc * C * (D / 2) * sizeof(float);
  const int64_t hbatch = (int64_t)(RC_HT_THREADS / (D / 8)) * RC_HK;
  const size_t hlds = hbytes + (size_t)hbatch * S * G + 16;   // table, a batch's code rows
  if (S >= 2 && S <= 4 && G % 2 == 0 && hbytes <= RC_LDS_MAX && hlds <= RC_LDS_BLOCK &&
      n_books <= 65535) {
    const int64_t batch = hbatch;
    int64_t nx = (256 + n_books - 1) / n_books;
    int64_t per = (n_per_book + nx - 1) / nx;
    per = (per + batch - 1) / batch * batch;
    nx = (n_per_book + per - 1) / per;
#define KVQ_RH(DD, SSV)                                                                       \
    if (D == DD && S == SSV) {                                                                \
      auto kern = reconstruct_half_kernel<DD, SSV, 2>;                                        \
      hipError_t e = hipFuncSetAttribute((const void*)kern,                                   \
                                         hipFuncAttributeMaxDynamicSharedMemorySize,          \
                                         (int)hlds);                                          \
      if (e != hipSuccess) return e;                                                          \
      kern<<<dim3((unsigned)nx, (unsigned)n_books), RC_HT_THREADS, hlds, s>>>(                \
          codes, cb, out, n_per_book, per, G, C, unrotate, sm.f, sm.n_scale, n_rows);         \
      return hipGetLastError();                                                               \
    }
    KVQ_RH(64, 2) KVQ_RH(128, 2) KVQ_RH(256, 2) KVQ_RH(64, 3) KVQ_RH(128, 3) KVQ_RH(256, 3)
    KVQ_RH(64, 4) KVQ_RH(128, 4) KVQ_RH(256, 4)
#undef KVQ_RH
  }
  if (cbytes <= RC_LDS_MAX && (S == 1 || S == 2 || (S == 4 && D < 256)) && n_books <= 65535) {
    // blocks per CU that fit the LDS, about 256 CUs' worth of blocks over the books
    const int per_cu = cbytes * 2 <= RC_LDS_BLOCK ? 2 : 1;
    const int64_t lvec = (int64_t)(RC_LDS_THREADS / 64) * (64 / (D / 8)) * RC_UNR;
    int64_t nx = (256 * per_cu + n_books - 1) / n_books;
    int64_t per = (n_per_book + nx - 1) / nx;
    per = (per + lvec - 1) / lvec * lvec;
    nx = (n_per_book + per - 1) / per;
    // the blocks' code rows go to LDS too when they fit beside the codebooks
    // (a 16-byte slack when a block's rows may start off a 16-byte boundary)
    const int64_t SG = (int64_t)S * G;
    const size_t slack = (n_per_book * SG) % 16 == 0 && (per * SG) % 16 == 0 ? 0 : 16;
    const size_t with_codes = cbytes + (size_t)per * SG + slack;
    const bool pre = with_codes <= RC_LDS_BLOCK / per_cu;
    const size_t ldsb = pre ? with_codes : cbytes;
#define KVQ_RL(DD, SSV)                                                                       \
    if (D == DD && S == SSV) {                                                               \
      auto kern = pre ? reconstruct_lds_kernel<DD, SSV, true>                                \
                      : reconstruct_lds_kernel<DD, SSV, false>;                              \
      hipError_t e = hipFuncSetAttribute((const void*)kern,                                  \
                                         hipFuncAttributeMaxDynamicSharedMemorySize,         \
                                         (int)ldsb);                                         \
      if (e != hipSuccess) return e;                                                         \
      kern<<<dim3((unsigned)nx, (unsigned)n_books), RC_LDS_THREADS, ldsb, s>>>(              \
          codes, cb, out, n_per_book, per, G, C, dsub, unrotate, sm.f, sm.n_scale, n_rows);  \
      return hipGetLastError();                                                              \
    }
    KVQ_RL(64, 1) KVQ_RL(128, 1) KVQ_RL(256, 1) KVQ_RL(64, 2) KVQ_RL(128, 2)
    KVQ_RL(64, 4) KVQ_RL(128, 4)
    // (D = 256 has an even group count, so its 2 and 4 stages take the half
    // tables or, with books over 128 KiB, the cache kernel)
#undef KVQ_RL
  }
  int64_t blocks = (n + vec_per_iter - 1) / vec_per_iter;
  if (blocks > 4096) blocks = 4096;
  auto kern = D == 64 ? reconstruct_kernel<64> : D == 128 ? reconstruct_kernel<128>
                                                          : reconstruct_kernel<256>;
  kern<<<dim3((unsigned)blocks), RC_THREADS, 0, s>>>(codes, cb, out, n_books, n_per_book, G, S, C,
                                                     dsub, unrotate, sm.f, sm.n_scale, n_rows);
  return hipGetLastError();
}

}  // namespace kvq
