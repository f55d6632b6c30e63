// K-means (Lloyd) fitting of residual product codebooks on a sample.
//
// "VeloxQuant-MLX 0.5.1", VecInfer section: the product-VQ codebooks are
// K-means codebooks trained before use (its allocator list names
// train_codebook); "VQKV" summary, 2. Methodology: the residual stage
// codebooks are trained.  Stage by stage, on the residuals the fitted earlier
// stages leave: n_iter times {assign every vector of the sample to its
// nearest entry; move every entry to the mean of its vectors (an entry with
// none keeps its value)}; then assign once more and subtract, which gives the
// next stage's residuals.
//
// Kernels, all on the caller's stream:
//   fit_prep_kernel      y = H_D (x / lambda) as float32 (kept for the whole
//                        call) and per group the largest |y| (bit pattern,
//                        atomic max);
//   assignment           the encode kernels themselves, run with the first
//                        s + 1 stages (their greedy chain runs the earlier,
//                        fitted stages and picks stage s's entry);
//   fit_accum_kernel     per (group, 32-dim slice, chunk of vectors): the
//                        stage-s residual y - sum_{t<s} C_t[z_t] rebuilt from
//                        the codes of that same assignment call (so the sums
//                        follow exactly the chain that chose z_s), summed per
//                        entry in LDS as 64-bit fixed point (ds_add_u64:
//                        integer adds, exact and independent of the order),
//                        stored as the chunk's partial sums;
//   fit_update_kernel    entry = (sum over chunks) * 2^-F / count in float64,
//                        rounded once to float32 (entries with no vector keep
//                        theirs);
//   fit_bound_kernel     after a stage's last assignment: per group the
//                        largest residual component, the next stage's bound.
// The kernels reading a stage's bound take the max over FIT_BCOPIES copies.
// Fixed point: F = 62 - ceil(log2 N) - e - m with the measured bound below 2^e
// and a margin m = 1 + ceil(log2 sqrt(dsub)).  The bound is measured on the
// chain of the stage's previous assignment call; a later call's chain can
// differ at a near tie (the assignment changes kernels between 4 and 5
// stages), and the margin covers any residual whose group norm stays within
// twice sqrt(dsub) times the bound, which such a chain gives.  Every term is
// below 2^(62 - ceil(log2 N)) (conversion clamps the shift there, so even a
// residual past the margin cannot overflow) and any sum of N of them below
// 2^62; a residual becomes a multiple of 2^-F exactly when |r| >= 2^(23-F),
// and is truncated toward zero (an error below 2^-F) otherwise.
#include "kvq_internal.h"

namespace kvq {

constexpr int FIT_CHUNK = 4096;      // vectors per accumulate block, at least
constexpr int FIT_MAX_CHUNKS = 64;   // chunks of the sample, at most
constexpr int FIT_DS = 32;           // dims per accumulate block (slice of a group)
// The per-group bounds are kept in this many copies, block b folding into
// copy b % FIT_BCOPIES (readers take the max over them): atomics on one
// address serialise, so spreading them keeps the bound off the critical path.
constexpr int FIT_BCOPIES = 32;

static inline size_t al256(size_t v) { return (v + 255) & ~(size_t)255; }

// vectors per accumulate chunk: FIT_CHUNK, or more so at most FIT_MAX_CHUNKS
static int64_t fit_chunk_len(int64_t n) {
  int64_t c = (n + FIT_MAX_CHUNKS - 1) / FIT_MAX_CHUNKS;
  c = (c + FIT_CHUNK - 1) / FIT_CHUNK * FIT_CHUNK;
  return c > FIT_CHUNK ? c : FIT_CHUNK;
}
static int64_t fit_chunks(int64_t n) {
  const int64_t c = fit_chunk_len(n);
  return n > 0 ? (n + c - 1) / c : 1;
}

FitLayout fit_layout(int D, int G, int S, int C, int64_t n) {
  FitLayout l{};
  const int dsub = D / G;
  size_t off = 0;
  l.resid = off;  off += al256((size_t)n * D * 4);
  l.codes = off;  off += al256((size_t)n * S * G);
  // the assignment of stage s runs the encode with s + 1 stages, on the MFMA
  // path (packed codebooks) whenever s + 1 <= 4: room for the longest such prefix
  l.pack = off;   off += al256(encode_workspace_bytes(D, G, S < 4 ? S : 4, C, 1));
  const int64_t nch = fit_chunks(n);
  l.acc = off;    off += al256((size_t)nch * G * C * dsub * 8);
  l.cnt = off;    off += al256((size_t)nch * G * C * 4);
  l.bound = off;  off += al256((size_t)(S + 1) * FIT_BCOPIES * G * 4);
  l.total = off;
  return l;
}

// bound: the stage's [FIT_BCOPIES][G] copies; margin: see the header
__device__ __forceinline__ int fit_fbits(const uint32_t* __restrict__ bound, int g, int G,
                                         int log2n, int margin) {
  uint32_t b = 0u;
  for (int i = 0; i < FIT_BCOPIES; ++i) b = bound[i * G + g] > b ? bound[i * G + g] : b;
  int e = 0;
  frexpf(__uint_as_float(b), &e);               // bound < 2^e (0 -> e = 0)
  return 62 - log2n - e - margin;
}

// x * 2^F as a 64-bit integer from the float's bits (integer ALU only): the
// mantissa shifted by exponent + F; exact when the result is a whole number
// (|x| >= 2^(23-F)), truncated toward zero below that.  The shift is clamped
// to shmax = 38 - ceil(log2 N), so every term is below 2^(62 - ceil(log2 N)).
__device__ __forceinline__ long long fit_fixed(float x, int F, int shmax) {
  const uint32_t u = __float_as_uint(x);
  const int ex = (int)((u >> 23) & 0xffu);
  const uint32_t man = (u & 0x7fffffu) | (ex ? 0x800000u : 0u);
  int sh = (ex ? ex : 1) - 150 + F;                     // x = man * 2^(ex - 150)
  sh = sh < shmax ? sh : shmax;
  long long t = sh >= 0 ? (long long)((unsigned long long)man << sh)
                        : (sh > -32 ? (long long)(man >> -sh) : 0ll);
  return (u >> 31) ? -t : t;
}

__global__ __launch_bounds__(256) void fit_clear_kernel(uint32_t* __restrict__ p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
    p[i] = 0u;
}

// L = D/8 lanes per row, 8 dims per lane (one group's dims when dsub >= 8).
template <int D, int XT>
__global__ __launch_bounds__(256) void fit_prep_kernel(const void* __restrict__ x,
                                                       float* __restrict__ r,
                                                       uint32_t* __restrict__ bound, int64_t n_seq,
                                                       int64_t seq_stride, int64_t n_rows, int dsub,
                                                       const float* __restrict__ smooth,
                                                       int64_t n_scale) {
  constexpr int L = D / 8;
  constexpr int RPP = 256 / L;
  constexpr int ESZ = XT == 0 ? 4 : 2;
  __shared__ uint32_t colmax[L];
  const int tid = threadIdx.x, lane = tid & 63;
  const int col = tid % L, rsub = tid / L;
  if (tid < L) colmax[tid] = 0u;
  __syncthreads();
  const int64_t n = n_seq * n_rows;
  uint32_t m = 0u;
  for (int64_t base = (int64_t)blockIdx.x * RPP; base < n; base += (int64_t)gridDim.x * RPP) {
    const int64_t v = base + rsub;
    const int64_t vl = v < n ? v : n - 1;               // every lane joins the butterfly
    const int64_t seq = vl / n_rows, row = vl - seq * n_rows;
    float val[8];
    load8<XT>(reinterpret_cast<const char*>(x) + ((seq * seq_stride + row) * D + col * 8) * ESZ,
              val);
    if (smooth != nullptr) {
      const float* lp = smooth + (seq % n_scale) * D + col * 8;
#pragma unroll
      for (int e = 0; e < 8; ++e) val[e] *= __builtin_amdgcn_rcpf(lp[e]);
    }
    hadamard_row<8, L>(val, lane);
    constexpr float sc = rsqrt_pow2(D);
#pragma unroll
    for (int e = 0; e < 8; ++e) val[e] *= sc;
    if (v < n) {
      float4* o = reinterpret_cast<float4*>(r + v * D + col * 8);
      o[0] = make_float4(val[0], val[1], val[2], val[3]);
      o[1] = make_float4(val[4], val[5], val[6], val[7]);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t a = __float_as_uint(val[e]) & 0x7fffffffu;
        m = a > m ? a : m;
      }
    }
  }
  atomicMax(&colmax[col], m);
  __syncthreads();
  const int cpg = dsub / 8;                             // columns per group
  if (tid < D / dsub) {
    uint32_t a = 0u;
    for (int c = tid * cpg; c < (tid + 1) * cpg; ++c) a = colmax[c] > a ? colmax[c] : a;
    if (a != 0u) atomicMax(bound + (blockIdx.x % FIT_BCOPIES) * (D / dsub) + tid, a);
  }
}

// grid (G * nslice, chunks).  Block: group g, dims [slice*DS, slice*DS + DS)
// of the group, vectors [chunk*len, (chunk+1)*len); each vector's stage-s
// residual over those dims (y minus the entries its earlier-stage codes
// chose, subtracted stage by stage in float32 as the encode does) goes to
// LDS sums[j][z] as fixed point, then the block stores its partial sums to
// part[chunk][g][j][c] (and counts to pcnt[chunk][g][c]).
template <int DS>
__global__ __launch_bounds__(256) void fit_accum_kernel(
    const float* __restrict__ y, const uint8_t* __restrict__ codes, int row_bytes, int s, int G,
    int C, int D, int dsub, const float* __restrict__ cb, int64_t n, int64_t len, int log2n,
    int margin, const uint32_t* __restrict__ bound, unsigned long long* __restrict__ part,
    uint32_t* __restrict__ pcnt) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  // [DS][C]: the lanes of one atomic instruction (same j, random entries z)
  // spread over the banks; [C][DS] would put them all DS * 8 bytes apart
  unsigned long long* sums = reinterpret_cast<unsigned long long*>(smem);
  uint32_t* counts = reinterpret_cast<uint32_t*>(smem + (size_t)C * DS * 8);
  const int nslice = dsub / DS;
  const int g = blockIdx.x / nslice, slice = blockIdx.x - g * nslice;
  const int tid = threadIdx.x;
  for (int i = tid; i < C * DS; i += 256) sums[i] = 0ull;
  for (int i = tid; i < C; i += 256) counts[i] = 0u;
  __syncthreads();
  const int F = fit_fbits(bound, g, G, log2n, margin);
  const int64_t n0 = (int64_t)blockIdx.y * len;
  const int64_t n1 = (n0 + len) < n ? (n0 + len) : n;
  const int d0 = g * dsub + slice * DS;
  // VB vectors per thread per pass, all their loads issued before any atomic
  // (indices past the end repeat the last vector; their atomics are skipped)
  constexpr int VB = DS == 32 ? 2 : 4;
  for (int64_t b = n0 + tid; b < n1; b += VB * 256) {
    int64_t vv[VB];
    int zz[VB];
    float4 a[VB][DS / 4];
#pragma unroll
    for (int k = 0; k < VB; ++k) {
      vv[k] = b + 256 * k < n1 ? b + 256 * k : n1 - 1;
      zz[k] = codes[vv[k] * row_bytes + s * G + g];
      const float4* rp = reinterpret_cast<const float4*>(y + vv[k] * D + d0);
#pragma unroll
      for (int q = 0; q < DS / 4; ++q) a[k][q] = rp[q];
    }
    for (int t = 0; t < s; ++t) {                       // the earlier stages' entries
      const float* cbt = cb + ((int64_t)t * G + g) * C * dsub + slice * DS;
#pragma unroll
      for (int k = 0; k < VB; ++k) {
        int zt = codes[vv[k] * row_bytes + t * G + g];
        zt = zt < C ? zt : C - 1;
        const float4* cp = reinterpret_cast<const float4*>(cbt + (int64_t)zt * dsub);
#pragma unroll
        for (int q = 0; q < DS / 4; ++q) {
          const float4 c4 = cp[q];
          a[k][q].x -= c4.x; a[k][q].y -= c4.y; a[k][q].z -= c4.z; a[k][q].w -= c4.w;
        }
      }
    }
#pragma unroll
    for (int k = 0; k < VB; ++k) {
      if (b + 256 * k >= n1) continue;
      const int z = zz[k] < C ? zz[k] : C - 1;
#pragma unroll
      for (int q = 0; q < DS / 4; ++q) {
        const float e4[4] = {a[k][q].x, a[k][q].y, a[k][q].z, a[k][q].w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const long long t = fit_fixed(e4[j], F, 38 - log2n);
          atomicAdd(&sums[(q * 4 + j) * C + z], (unsigned long long)t);
        }
      }
      if (slice == 0) atomicAdd(&counts[z], 1u);
    }
  }
  __syncthreads();
  unsigned long long* pp = part + (((int64_t)blockIdx.y * G + g) * dsub + slice * DS) * C;
  for (int i = tid; i < C * DS; i += 256) pp[i] = sums[i];
  if (slice == 0) {
    uint32_t* pc = pcnt + ((int64_t)blockIdx.y * G + g) * C;
    for (int c = tid; c < C; c += 256) pc[c] = counts[c];
  }
}

// grid (G, dsub), one entry c per thread (C <= 256): the chunks' partial sums
// and counts added in chunk order (integers: exact).
__global__ __launch_bounds__(256) void fit_update_kernel(
    float* __restrict__ cb_s, int G, int C, int dsub, int log2n, int margin, int64_t nch,
    const uint32_t* __restrict__ bound, const unsigned long long* __restrict__ part,
    const uint32_t* __restrict__ pcnt) {
  const int g = blockIdx.x, j = blockIdx.y, c = threadIdx.x;
  if (c >= C) return;
  const int F = fit_fbits(bound, g, G, log2n, margin);
  unsigned long long sum = 0ull;
  uint32_t k = 0u;
  for (int64_t h = 0; h < nch; ++h) {
    sum += part[((h * G + g) * dsub + j) * C + c];
    k += pcnt[(h * G + g) * C + c];
  }
  if (k != 0u)
    cb_s[((int64_t)g * C + c) * dsub + j] = (float)(ldexp((double)(long long)sum, -F) / (double)k);
}

// Per group, the largest component of y - sum_{t<=s} C_t[z_t] over the
// vectors (the residual stage s + 1 starts from), from the codes of stage s's
// last assignment (stages 0..s in each row).
template <int D>
__global__ __launch_bounds__(256) void fit_bound_kernel(
    const float* __restrict__ y, const uint8_t* __restrict__ codes, int row_bytes, int s, int G,
    int C, int dsub, const float* __restrict__ cb, int64_t n, uint32_t* __restrict__ bound_next) {
  constexpr int L = D / 8;
  constexpr int RPP = 256 / L;
  __shared__ uint32_t colmax[L];
  const int tid = threadIdx.x;
  const int col = tid % L, rsub = tid / L;
  if (tid < L) colmax[tid] = 0u;
  __syncthreads();
  const int g = col * 8 / dsub, j0 = col * 8 - g * dsub;
  uint32_t m = 0u;
  for (int64_t base = (int64_t)blockIdx.x * RPP; base < n; base += (int64_t)gridDim.x * RPP) {
    const int64_t v = base + rsub;
    if (v >= n) continue;
    const float4* rp = reinterpret_cast<const float4*>(y + v * D + col * 8);
    float4 a = rp[0], b = rp[1];
    for (int t = 0; t <= s; ++t) {
      int z = codes[v * row_bytes + t * G + g];
      z = z < C ? z : C - 1;
      const float4* cp =
          reinterpret_cast<const float4*>(cb + (((int64_t)t * G + g) * C + z) * dsub + j0);
      const float4 c0 = cp[0], c1 = cp[1];
      a.x -= c0.x; a.y -= c0.y; a.z -= c0.z; a.w -= c0.w;
      b.x -= c1.x; b.y -= c1.y; b.z -= c1.z; b.w -= c1.w;
    }
    const float e8[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t t = __float_as_uint(e8[e]) & 0x7fffffffu;
      m = t > m ? t : m;
    }
  }
  atomicMax(&colmax[col], m);
  __syncthreads();
  const int cpg = dsub / 8;
  if (tid < D / dsub) {
    uint32_t a = 0u;
    for (int c = tid * cpg; c < (tid + 1) * cpg; ++c) a = colmax[c] > a ? colmax[c] : a;
    if (a != 0u) atomicMax(bound_next + (blockIdx.x % FIT_BCOPIES) * (D / dsub) + tid, a);
  }
}

static int ceil_log2_i64(int64_t v) {
  int k = 0;
  while (((int64_t)1 << k) < v) ++k;
  return k;
}

static int64_t grid_rows(int64_t n, int D) {
  const int64_t rpp = 256 / (D / 8);
  int64_t b = (n + rpp - 1) / rpp;
  return b < 2048 ? (b > 0 ? b : 1) : 2048;
}

hipError_t launch_codebook_fit(const void* x, int xt, int D, int G, int S, int C, int64_t n_seq,
                               int64_t seq_stride, int64_t n_rows, Smooth sm, int n_iter,
                               float* cb, void* ws, hipStream_t st) {
  const int64_t n = n_seq * n_rows;
  if (n == 0) return hipSuccess;
  const int dsub = D / G;
  const FitLayout lay = fit_layout(D, G, S, C, n);
  uint8_t* w = reinterpret_cast<uint8_t*>(ws);
  float* r = reinterpret_cast<float*>(w + lay.resid);
  uint8_t* codes = w + lay.codes;
  void* pack = w + lay.pack;
  unsigned long long* acc = reinterpret_cast<unsigned long long*>(w + lay.acc);
  uint32_t* cnt = reinterpret_cast<uint32_t*>(w + lay.cnt);
  uint32_t* bound = reinterpret_cast<uint32_t*>(w + lay.bound);
  const int log2n = ceil_log2_i64(n);

  // the bounds start at zero (the partial sums are overwritten by every pass)
  const int64_t nclear = (int64_t)(lay.total - lay.bound) / 4;
  fit_clear_kernel<<<dim3((unsigned)((nclear + 255) / 256 < 1024 ? (nclear + 255) / 256 : 1024)),
                     dim3(256), 0, st>>>(bound, nclear);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;

  const int64_t rb = grid_rows(n, D);
#define KVQ_PREP(DD, XX)                                                                    \
  if (D == DD && xt == XX)                                                                 \
    fit_prep_kernel<DD, XX><<<dim3((unsigned)rb), dim3(256), 0, st>>>(                      \
        x, r, bound, n_seq, seq_stride, n_rows, dsub, sm.f, sm.n_scale);
  KVQ_PREP(64, 0) KVQ_PREP(64, 1) KVQ_PREP(64, 2)
  KVQ_PREP(128, 0) KVQ_PREP(128, 1) KVQ_PREP(128, 2)
  KVQ_PREP(256, 0) KVQ_PREP(256, 1) KVQ_PREP(256, 2)
#undef KVQ_PREP
  e = hipGetLastError();
  if (e != hipSuccess) return e;

  const int ds = dsub < FIT_DS ? dsub : FIT_DS;
  const int margin = 1 + (ceil_log2_i64(dsub) + 1) / 2;  // 1 + ceil(log2 sqrt(dsub))
  const int nslice = dsub / ds;
  const int64_t clen = fit_chunk_len(n);
  const int64_t chunks = fit_chunks(n);
  const size_t alds = (size_t)C * ds * 8 + (size_t)C * 4;
  for (int s = 0; s < S; ++s) {
    const int sp = s + 1;                               // stages run by the assignment
    const int row_bytes = sp * G;
    float* cb_s = cb + (size_t)s * G * C * dsub;
    const uint32_t* bs = bound + (size_t)s * FIT_BCOPIES * G;
    const bool last = s == S - 1;
    for (int it = 0; it < n_iter + (last ? 0 : 1); ++it) {
      e = launch_encode(x, xt, D, G, sp, C, 1, n_seq, seq_stride, n_rows, cb, codes, n_rows, 0, 0,
                        0, 0, pack, sm, st);
      if (e != hipSuccess) return e;
      if (it == n_iter) break;                          // final assignment of a non-last stage
#define KVQ_ACC(DSV)                                                                         \
  if (ds == DSV) {                                                                          \
    e = hipFuncSetAttribute((const void*)fit_accum_kernel<DSV>,                             \
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)alds);         \
    if (e != hipSuccess) return e;                                                          \
    fit_accum_kernel<DSV><<<dim3((unsigned)(G * nslice), (unsigned)chunks), dim3(256), alds, \
                            st>>>(r, codes, row_bytes, s, G, C, D, dsub, cb, n, clen, log2n, \
                                  margin, bs, acc, cnt);                                    \
  }
      KVQ_ACC(8) KVQ_ACC(16) KVQ_ACC(32)
#undef KVQ_ACC
      e = hipGetLastError();
      if (e != hipSuccess) return e;
      fit_update_kernel<<<dim3(G, dsub), dim3(256), 0, st>>>(cb_s, G, C, dsub, log2n, margin,
                                                             chunks, bs, acc, cnt);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
    if (!last) {
      auto kern = D == 64 ? fit_bound_kernel<64>
                          : D == 128 ? fit_bound_kernel<128> : fit_bound_kernel<256>;
      kern<<<dim3((unsigned)rb), dim3(256), 0, st>>>(r, codes, row_bytes, s, G, C, dsub, cb, n,
                                                      bound + (size_t)(s + 1) * FIT_BCOPIES * G);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  }
  return hipSuccess;
}

}  // namespace kvq
