// K2 -- encode: Walsh-Hadamard rotation, then per group S greedy residual
// stages of nearest-codeword search, codes stored as bytes.
//
// Steps ("VQKV" summary, 2. Methodology, Residual Simple Vector
// Quantization; "VeloxQuant-MLX 0.5.1", VecInfer product VQ after a
// Walsh-Hadamard rotation, one codebook per sub-vector):
//   y = H_D x; for each group g: r = y_g; for s: z = argmin_c |r - C_sg[c]|^2,
//   r -= C_sg[z].
//
// Two kernels:
//   * encode_mfma_kernel -- D = 128, dsub = 8, C = 256, 2-byte input.  The
//     distance contraction e[c][n] = |c|^2 + beta_n - 2 c.r_n is a dense GEMM
//     on MFMA (v_mfma_f32_32x32x16_bf16).  Exact-enough products come from
//     split operands: r = r_hi + r_lo and c = c_hi + c_lo in bf16,
//     -2(c_hi.r_hi + c_lo.r_hi + c_hi.r_lo) over K = 24 slots, plus |c|^2 as
//     three bf16 pieces and beta_n = |r_n|^2 rounded up to bf16 over the
//     remaining slots, accumulated in fp32.  The argmin packs the codeword
//     index into the 8 low mantissa bits of the (non-negative) distance and
//     takes a signed integer minimum (v_min3_i32), which perturbs distances by
//     at most 2^-15 relative -- inside the 1e-4 near-tie band.
//   * encode_generic_kernel -- any D in {64,128,256}, dsub in {8..128}, any
//     C <= 256, any input type: plain fp32 distances on the vector ALUs.
#include "kvq_internal.h"

namespace kvq {

// ============================================================ codebook pack
// Workspace layout for the MFMA kernel, per (book, g, s), 20480 bytes:
//   +0     hi [256][8] bf16   = bf16(-2 c)
//   +4096  lo [256][8] bf16   = bf16(-2 (c - bf16(c)))
//   +8192  nrm[256][8] bf16   = (n1, n2, n3, 1, 0, 0, 0, 0), n1+n2+n3 ~ |c|^2
//   +12288 f32[256][8]        = c (for the residual update)
// ordered [book][g][s] so a group's S stage blocks are contiguous.
constexpr int PACK_BYTES = 20480;

__global__ void pack_codebooks_kernel(const float* __restrict__ cb, uint8_t* __restrict__ ws,
                                      int64_t n_books, int S, int G) {
  const int64_t total = n_books * S * G * 256;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int c = (int)(i & 255);
    int64_t t = i >> 8;
    const int g = (int)(t % G); t /= G;
    const int s = (int)(t % S); t /= S;
    const int64_t book = t;
    const float* src = cb + ((((book * S) + s) * G + g) * 256 + c) * 8;
    uint8_t* dst = ws + ((book * G + g) * S + s) * (int64_t)PACK_BYTES;
    float v[8];
    double n = 0.0;
#pragma unroll
    for (int j = 0; j < 8; ++j) { v[j] = src[j]; n += (double)v[j] * (double)v[j]; }
    uint32_t hi[4], lo[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      float a = v[2 * k], b = v[2 * k + 1];
      uint32_t ha = f32_to_bf16_rne(a), hb = f32_to_bf16_rne(b);
      hi[k] = f32_to_bf16_rne(-2.0f * a) | (f32_to_bf16_rne(-2.0f * b) << 16);
      float la = a - bf16_bits_to_f32(ha), lb = b - bf16_bits_to_f32(hb);
      lo[k] = f32_to_bf16_rne(-2.0f * la) | (f32_to_bf16_rne(-2.0f * lb) << 16);
    }
    const float nf = (float)n;
    const uint32_t n1 = f32_to_bf16_rne(nf);
    const double r1 = n - (double)bf16_bits_to_f32(n1);
    const uint32_t n2 = f32_to_bf16_rne((float)r1);
    const double r2 = r1 - (double)bf16_bits_to_f32(n2);
    const uint32_t n3 = f32_to_bf16_rne((float)r2);
    const uint32_t one = 0x3F80u;
    reinterpret_cast<uint4*>(dst + 0)[c] = make_uint4(hi[0], hi[1], hi[2], hi[3]);
    reinterpret_cast<uint4*>(dst + 4096)[c] = make_uint4(lo[0], lo[1], lo[2], lo[3]);
    reinterpret_cast<uint4*>(dst + 8192)[c] = make_uint4(n1 | (n2 << 16), n3 | (one << 16), 0u, 0u);
    float4* f = reinterpret_cast<float4*>(dst + 12288) + 2 * c;
    f[0] = make_float4(v[0], v[1], v[2], v[3]);
    f[1] = make_float4(v[4], v[5], v[6], v[7]);
  }
}

// ================================================================ MFMA path
constexpr int MF_SCRATCH = 4096;            // per-wave transpose scratch (bytes)

// Waves per block (64 vectors each) and LDS bytes of one group's codebook
// buffer (the last stage's fp32 copy is never read: no residual update
// follows it).  Up to two stages, blocks of 4 waves with two codebook buffers
// fit twice per CU, so one block's row loads, rotation and barrier waits
// overlap the other's argmin; four stages need the whole LDS for one block.
template <int S> constexpr int mf_waves() { return S <= 2 ? 4 : 8; }
template <int S> constexpr int mf_buf() { return (S - 1) * 20480 + 12288; }

// Row address (in elements) of vector n of a book.
__device__ __forceinline__ int64_t row_elem(int64_t book, int64_t n, int64_t n_rows, int64_t n_seq,
                                            int64_t seq_stride) {
  const int64_t seq = n / n_rows, row = n - seq * n_rows;
  return ((book * n_seq + seq) * seq_stride + row) * 128;
}

// Code row of vector n of a book: rows [code_row0, code_row0 + n_rows) of a
// sequence whose code rows are code_stride apart.
__device__ __forceinline__ int64_t code_row(int64_t book, int64_t n, int64_t n_rows, int64_t n_seq,
                                            int64_t code_stride, int64_t code_row0) {
  const int64_t seq = n / n_rows, row = n - seq * n_rows;
  return (book * n_seq + seq) * code_stride + code_row0 + row;
}

// Copy one group's S packed stage blocks (S * 20480 contiguous bytes) from
// global memory straight into LDS with global_load_lds_dwordx4: each
// instruction moves 64 lanes x 16 bytes into 1 KiB of LDS at a wave-uniform
// base.  Completion is awaited with wait_vmem().
template <int S>
__device__ __forceinline__ void stage_group(const uint8_t* src, uint8_t* dst, int wave, int lane) {
  // 20 KiB per stage, except 12 KiB for the last one (mf_buf)
  constexpr int PIECES = 20 * (S - 1) + 12;
  constexpr int W = mf_waves<S>();
#pragma unroll
  for (int k = 0; k < (PIECES + W - 1) / W; ++k) {
    const int piece = k * W + wave;                      // wave-uniform
    if (piece < PIECES) {
      const int st = piece / 20 < S - 1 ? piece / 20 : S - 1;
      const int off = st * PACK_BYTES + (piece - 20 * st) * 1024;
      __builtin_amdgcn_global_load_lds(src + off + lane * 16,
                                       (__attribute__((address_space(3))) void*)(dst + off),
                                       16, 0, 0);
    }
  }
}

__device__ __forceinline__ void wait_vmem() {
  __builtin_amdgcn_s_waitcnt(0x0f70);                    // vmcnt(0)
}

template <int S, int XT, int GS>   // GS: 1 = a block codes all 16 groups of its tile;
                                   // 0 = gsplit blocks share them (runtime)
__global__ __launch_bounds__(64 * mf_waves<S>(), 8 / mf_waves<S>()) void encode_mfma_kernel(
    const uint16_t* __restrict__ x, const uint8_t* __restrict__ packed, uint8_t* __restrict__ codes,
    int64_t n_seq, int64_t seq_stride, int64_t n_rows, int64_t code_stride, int64_t code_row0,
    int64_t tiles_per_book, int pre_rotated, const float* __restrict__ smooth, int64_t n_scale,
    int gsplit) {
  constexpr int G = 16;
  constexpr int SG = S * G;
  // GS = 0 (small batches): gsplit blocks per tile, each rotating the tile
  // itself and coding the groups [g_lo, g_hi) -- more blocks in flight for a
  // batch too small to give every SIMD two waves.
  // LDS: two buffers of one group's S stage blocks (double buffering); the
  // per-wave transpose scratch of the tile's input rows aliases them, since
  // it is dead before the first codebook load is issued.
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int h = lane >> 5;                                // lane half
  uint8_t* scratch = smem + wave * MF_SCRATCH;

  const int gsp = GS == 1 ? 1 : gsplit;
  const int g_lo = GS == 1 ? 0 : (int)(blockIdx.x % gsp) * (G / gsp);
  const int g_hi = GS == 1 ? G : g_lo + G / gsp;
  const int64_t bt = blockIdx.x / gsp;
  const int64_t book = bt / tiles_per_book;
  const int64_t tile = bt - book * tiles_per_book;
  const int64_t n_per_book = n_seq * n_rows;
  constexpr int TILE = 64 * mf_waves<S>();
  constexpr int BUF = mf_buf<S>();
  const int64_t v_own = tile * TILE + wave * 64 + lane;              // vector this lane owns
  const bool live = v_own < n_per_book;
  const int64_t v_ld = live ? v_own : (n_per_book - 1);
  const int64_t my_row = row_elem(book, v_ld, n_rows, n_seq, seq_stride);

  // ---- load the lane's row through a transposing LDS scratch (coalesced reads)
  uint32_t xw[64];                                       // 128 bf16/f16 elements, packed pairs
#pragma unroll
  for (int q = 0; q < 4; ++q) {                         // 16 rows per round
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int rloc = 4 * k + (lane >> 4);             // row within the round
      const int c = lane & 15;                          // 16-byte chunk within the row
      const int src_lane = 16 * q + rloc;
      const int64_t rb = (int64_t)__shfl((long long)my_row, src_lane);
      const uint4 w = *reinterpret_cast<const uint4*>(x + rb + c * 8);
      reinterpret_cast<uint4*>(scratch)[rloc * 16 + (c ^ rloc)] = w;
    }
    __syncthreads();                                    // round's rows are in LDS
    if ((lane >> 4) == q) {
      const int rloc = lane & 15;
#pragma unroll
      for (int c = 0; c < 16; ++c) {
        const uint4 w = reinterpret_cast<const uint4*>(scratch)[rloc * 16 + (c ^ rloc)];
        xw[4 * c + 0] = w.x; xw[4 * c + 1] = w.y; xw[4 * c + 2] = w.z; xw[4 * c + 3] = w.w;
      }
    }
    __syncthreads();                                    // scratch free for the next round
  }

  const uint8_t* pk_book = packed + book * (int64_t)G * S * PACK_BYTES;
  // the first group's codebooks load while the rotation runs
  stage_group<S>(pk_book + (int64_t)g_lo * S * PACK_BYTES, smem + (g_lo & 1) * mf_buf<S>(), wave,
                 lane);

  // ---- y = H x (or x itself when pre-rotated), float32 in registers
  float y[128];
#pragma unroll
  for (int i = 0; i < 64; ++i) {
    if constexpr (XT == 1) {
      y[2 * i] = bf16_lo(xw[i]);
      y[2 * i + 1] = bf16_hi(xw[i]);
    } else {
      y[2 * i] = f16_bits_to_f32(xw[i]);
      y[2 * i + 1] = f16_bits_to_f32(xw[i] >> 16);
    }
  }
  if (smooth != nullptr) {
    // dual transform: channel i divided by the sequence's factor (times its
    // reciprocal, within 1 ulp) ahead of the rotation
    const float4* lp = reinterpret_cast<const float4*>(
        smooth + (book * n_scale + (v_ld / n_rows) % n_scale) * 128);
#pragma unroll
    for (int c = 0; c < 32; ++c) {
      const float4 l = lp[c];
      y[4 * c + 0] *= __builtin_amdgcn_rcpf(l.x);
      y[4 * c + 1] *= __builtin_amdgcn_rcpf(l.y);
      y[4 * c + 2] *= __builtin_amdgcn_rcpf(l.z);
      y[4 * c + 3] *= __builtin_amdgcn_rcpf(l.w);
    }
  }
  if (!pre_rotated) {
#pragma unroll
    for (int hstep = 1; hstep < 128; hstep <<= 1) {
#pragma unroll
      for (int i = 0; i < 128; ++i) {
        if ((i & hstep) == 0) {
          const float a = y[i], b = y[i + hstep];
          y[i] = a + b;
          y[i + hstep] = a - b;
        }
      }
    }
    constexpr float sc = 0.08838834764831845f;
#pragma unroll
    for (int i = 0; i < 128; ++i) y[i] *= sc;
  }

  uint32_t cw[SG / 4];
#pragma unroll
  for (int i = 0; i < SG / 4; ++i) cw[i] = 0u;
  wait_vmem();
  __syncthreads();                                        // group 0 staged

  const int m_lane = lane & 31;
  // 0xffffff00 held in a vector register (an opaque value, so the compiler
  // keeps it as the v_and_or_b32 mask operand instead of a literal)
  uint32_t keep_hi = 0xffffff00u;
  asm volatile("" : "+v"(keep_hi));

#pragma unroll
  for (int g = 0; g < G; ++g) {
    if constexpr (GS != 1) {
      if (g < g_lo || g >= g_hi) continue;               // block-uniform
    }
    const uint8_t* cbs = smem + (g & 1) * BUF;
    // ---- the next group's codebooks stream into the other buffer meanwhile
    if (g + 1 < g_hi) stage_group<S>(pk_book + (int64_t)(g + 1) * S * PACK_BYTES,
                                     smem + ((g + 1) & 1) * BUF, wave, lane);

    float r[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) r[j] = y[8 * g + j];

#pragma unroll
    for (int s = 0; s < S; ++s) {
      const uint8_t* cbs_s = cbs + s * PACK_BYTES;
      // ---- B operands: r_hi, r_lo as bf16, beta = |r|^2 rounded up to bf16
      uint32_t hi[4], lo[4], nr[4];
      float nrm = 0.0f;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float a = r[2 * k], b = r[2 * k + 1];
        hi[k] = cvt_pk_bf16(a, b);
        const float la = a - bf16_lo(hi[k]), lb = b - bf16_hi(hi[k]);
        lo[k] = cvt_pk_bf16(la, lb);
        nrm = __builtin_fmaf(a, a, nrm);
        nrm = __builtin_fmaf(b, b, nrm);
      }
      const uint32_t beta = (__float_as_uint(nrm) + 0xffffu) >> 16;   // round up (nrm >= 0)
      nr[0] = 0x3F803F80u;
      nr[1] = 0x3F80u | (beta << 16);
      nr[2] = 0u;
      nr[3] = 0u;
      // Exchange so that both lane halves feed the columns of each 32-vector tile.
      uint32_t b1t0[4], b1t1[4], b2t0[4], b2t1[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        auto p = __builtin_amdgcn_permlane32_swap(hi[k], hi[k], false, false);
        b1t0[k] = p[0]; b1t1[k] = p[1];
        auto q2 = __builtin_amdgcn_permlane32_swap(lo[k], nr[k], false, false);
        b2t0[k] = q2[0]; b2t1[k] = q2[1];
      }
      bf16x8_t B1T0, B1T1, B2T0, B2T1;
      __builtin_memcpy(&B1T0, b1t0, 16); __builtin_memcpy(&B1T1, b1t1, 16);
      __builtin_memcpy(&B2T0, b2t0, 16); __builtin_memcpy(&B2T1, b2t1, 16);

      int best0 = 0x7fffffff, best1 = 0x7fffffff;
      // One codeword tile = 32 codewords x (2 x 32 vectors): two MFMAs per
      // 32-vector half (A1.B1 then A2.B2 accumulated), then the argmin.
      auto load_a = [&](int t, bf16x8_t& A1, bf16x8_t& A2) {
        const int m = 32 * t + m_lane;
        const uint4 a1 = *reinterpret_cast<const uint4*>(cbs_s + h * 4096 + m * 16);
        const uint4 a2 = *reinterpret_cast<const uint4*>(cbs_s + h * 8192 + m * 16);
        __builtin_memcpy(&A1, &a1, 16);
        __builtin_memcpy(&A2, &a2, 16);
      };
      // The packed index (32t | row) comes from a scalar register, so each
      // candidate costs one v_and_or_b32; accumulator register i holds codeword
      // row 8*(i/4) + 4*h + (i%4) of the tile (h is or-ed in after the loop).
      // One call reduces 8 of a tile's 16 candidates.
      auto reduce8 = [&](int t, const f32x16_t& c, int& best, int lo) {
        const uint32_t tb = (uint32_t)__builtin_amdgcn_readfirstlane(t << 5);
#pragma unroll
        for (int i = lo; i < lo + 8; ++i) {
          const uint32_t idx = tb | (uint32_t)(8 * (i >> 2) + (i & 3));
          best = min(best, (int)((__float_as_uint(c[i]) & keep_hi) | idx));
        }
      };
      // The halves staggered: one half's MFMA pair is issued before the other
      // half's previous tile is reduced, so the reduction never waits for the
      // MFMAs just issued.
      bf16x8_t A1, A2;
      f32x16_t acc0, acc1;
      const f32x16_t zero = {0};
      load_a(0, A1, A2);
      acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A1, B1T0, zero, 0, 0, 0);
      acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A2, B2T0, acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A1, B1T1, zero, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A2, B2T1, acc1, 0, 0, 0);
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const bool more = t + 1 < 8;
        if (more) load_a(t + 1, A1, A2);
        reduce8(t, acc0, best0, 0);
        reduce8(t, acc0, best0, 8);
        if (more) {
          acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A1, B1T0, zero, 0, 0, 0);
          acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A2, B2T0, acc0, 0, 0, 0);
        }
        reduce8(t, acc1, best1, 0);
        reduce8(t, acc1, best1, 8);
        if (more) {
          acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A1, B1T1, zero, 0, 0, 0);
          acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A2, B2T1, acc1, 0, 0, 0);
        }
      }
      best0 |= h << 2;
      best1 |= h << 2;
      auto bb = __builtin_amdgcn_permlane32_swap((uint32_t)best0, (uint32_t)best1, false, false);
      const int mine = min((int)bb[0], (int)bb[1]);
      const uint32_t z = (uint32_t)mine & 255u;
      {
        const int pos = s * G + g;                         // code byte (s, g) of the row
        cw[pos >> 2] |= z << (8 * (pos & 3));
      }
      if (s + 1 < S) {
        const float4* cf = reinterpret_cast<const float4*>(cbs_s + 12288 + z * 32);
        const float4 c0 = cf[0], c1 = cf[1];
        r[0] -= c0.x; r[1] -= c0.y; r[2] -= c0.z; r[3] -= c0.w;
        r[4] -= c1.x; r[5] -= c1.y; r[6] -= c1.z; r[7] -= c1.w;
      }
    }
    // own loads of the next group landed; after the barrier every wave's have,
    // and every wave is done reading this group's buffer
    wait_vmem();
    __syncthreads();
  }

  if (live) {
    uint8_t* row = codes + code_row(book, v_own, n_rows, n_seq, code_stride, code_row0) * SG;
    if constexpr (GS == 1) {
      uint4* dst = reinterpret_cast<uint4*>(row);
#pragma unroll
      for (int i = 0; i < SG / 16; ++i)
        dst[i] = make_uint4(cw[4 * i], cw[4 * i + 1], cw[4 * i + 2], cw[4 * i + 3]);
    } else {                                             // this block's code bytes only
#pragma unroll
      for (int s = 0; s < S; ++s)
#pragma unroll
        for (int g = 0; g < G; ++g) {
          const int pos = s * G + g;
          if (g >= g_lo && g < g_hi) row[pos] = (uint8_t)(cw[pos >> 2] >> (8 * (pos & 3)));
        }
    }
  }
}

// ============================================================= generic path
constexpr int GEN_TILE = 64;       // vectors per block

template <int D, int DSUB>
__global__ __launch_bounds__(256) void encode_generic_kernel(
    const void* __restrict__ x, int xt, const float* __restrict__ cb, uint8_t* __restrict__ codes,
    int64_t n_seq, int64_t seq_stride, int64_t n_rows, int64_t code_stride, int64_t code_row0,
    int64_t tiles_per_book, int S, int C, int pre_rotated, const float* __restrict__ smooth,
    int64_t n_scale) {
  constexpr int G = D / DSUB;
  constexpr int L = D / 8;
  constexpr int ROWS_PER_WAVE = 64 / L;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  float* ys = reinterpret_cast<float*>(smem);                         // [GEN_TILE][D]
  uint8_t* cs = smem + GEN_TILE * D * sizeof(float);                  // [GEN_TILE][S*G]
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t book = blockIdx.x / tiles_per_book;
  const int64_t tile = blockIdx.x - book * tiles_per_book;
  const int64_t n_per_book = n_seq * n_rows;
  const int64_t v0 = tile * GEN_TILE;
  const int SG = S * G;
  const int esz = xt == 0 ? 4 : 2;
  const char* xb = reinterpret_cast<const char*>(x);

  // ---- rotate the tile into LDS: L lanes per row, 8 elements per lane
  for (int rb = wave * ROWS_PER_WAVE; rb < GEN_TILE; rb += 4 * ROWS_PER_WAVE) {
    const int rl = rb + lane / L;
    const int col = lane % L;
    int64_t v = v0 + rl;
    if (v >= n_per_book) v = n_per_book - 1;
    const int64_t seq = v / n_rows, row = v - seq * n_rows;
    const int64_t e = ((book * n_seq + seq) * seq_stride + row) * D + col * 8;
    float val[8];
    if (xt == 0) load8<0>(xb + e * esz, val);
    else if (xt == 1) load8<1>(xb + e * esz, val);
    else load8<2>(xb + e * esz, val);
    if (smooth != nullptr) {            // dual transform: divide by the factor row
      const float* lp = smooth + (book * n_scale + seq % n_scale) * D + col * 8;
#pragma unroll
      for (int i = 0; i < 8; ++i) val[i] *= __builtin_amdgcn_rcpf(lp[i]);
    }
    if (!pre_rotated) {
      hadamard_row<8, L>(val, lane);
      constexpr float sc = rsqrt_pow2(D);
#pragma unroll
      for (int i = 0; i < 8; ++i) val[i] *= sc;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) ys[rl * D + col * 8 + i] = val[i];
  }
  __syncthreads();

  // ---- per (vector, group) greedy residual chain; a wave shares one group
  for (int g = wave; g < G; g += 4) {
    const int vl = lane;                  // GEN_TILE == 64
    float r[DSUB];
#pragma unroll
    for (int j = 0; j < DSUB; ++j) r[j] = ys[vl * D + g * DSUB + j];
    for (int s = 0; s < S; ++s) {
      const float* cbg = cb + ((book * S + s) * G + g) * (int64_t)C * DSUB;
      float best = __builtin_inff();
      int bz = 0;
      for (int c = 0; c < C; ++c) {
        const float* cc = cbg + c * DSUB;
        float d = 0.0f;
#pragma unroll
        for (int j = 0; j < DSUB; ++j) {
          const float t = r[j] - cc[j];
          d = __builtin_fmaf(t, t, d);
        }
        if (d < best) { best = d; bz = c; }
      }
      cs[vl * SG + s * G + g] = (uint8_t)bz;
      const float* cz = cbg + bz * DSUB;
#pragma unroll
      for (int j = 0; j < DSUB; ++j) r[j] -= cz[j];
    }
  }
  __syncthreads();

  // ---- write the tile's code rows
  const int64_t nv = (n_per_book - v0) < GEN_TILE ? (n_per_book - v0) : GEN_TILE;
  for (int i = threadIdx.x; i < nv * SG; i += 256) {
    const int vl = i / SG;
    codes[code_row(book, v0 + vl, n_rows, n_seq, code_stride, code_row0) * SG + (i - vl * SG)] = cs[i];
  }
}

// ================================================================ launchers
size_t encode_workspace_bytes(int D, int G, int S, int C, int64_t n_books) {
  if (D == 128 && G == 16 && C == 256 && S <= 4) return (size_t)n_books * G * S * PACK_BYTES;
  return 0;
}

bool encode_mfma_eligible(int D, int G, int S, int C, int xt) {
  return D == 128 && G == 16 && C == 256 && S >= 1 && S <= 4 && (xt == 1 || xt == 2);
}

template <int S, int XT>
static hipError_t launch_mfma_t(const void* x, const uint8_t* packed, uint8_t* codes,
                                int64_t n_books, int64_t n_seq, int64_t seq_stride, int64_t n_rows,
                                int64_t code_stride, int64_t code_row0, int pre_rotated,
                                Smooth sm, hipStream_t st) {
  const int64_t n_per_book = n_seq * n_rows;
  constexpr int TILE = 64 * mf_waves<S>();
  const int64_t tiles = (n_per_book + TILE - 1) / TILE;
  // a small batch (a window flush, a codebook-fitting sample) shares each
  // tile's 16 groups out over gsplit blocks: the fewest that give the CUs'
  // SIMDs two waves each (512 blocks), at most 16
  const int64_t blocks = tiles * n_books;
  int gs = 1;
  while (gs < 16 && blocks * gs < 512) gs *= 2;
  size_t lds = (size_t)2 * mf_buf<S>();                    // two codebook buffers
  if (lds < (size_t)mf_waves<S>() * MF_SCRATCH) lds = (size_t)mf_waves<S>() * MF_SCRATCH;
  auto kern = gs > 1 ? encode_mfma_kernel<S, XT, 0> : encode_mfma_kernel<S, XT, 1>;
  hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                                     (int)lds);
  if (e != hipSuccess) return e;
  kern<<<dim3((unsigned)(blocks * gs)), dim3(64 * mf_waves<S>()), lds, st>>>(
      reinterpret_cast<const uint16_t*>(x), packed, codes, n_seq, seq_stride, n_rows, code_stride,
      code_row0, tiles, pre_rotated, sm.f, sm.n_scale, gs);
  return hipGetLastError();
}

template <int D, int DSUB>
static hipError_t launch_generic_t(const void* x, int xt, const float* cb, uint8_t* codes,
                                   int64_t n_books, int64_t n_seq, int64_t seq_stride,
                                   int64_t n_rows, int64_t code_stride, int64_t code_row0, int S,
                                   int C, int pre_rotated, Smooth sm, hipStream_t st) {
  const int64_t n_per_book = n_seq * n_rows;
  const int64_t tiles = (n_per_book + GEN_TILE - 1) / GEN_TILE;
  const int G = D / DSUB;
  const size_t lds = (size_t)GEN_TILE * D * sizeof(float) + (size_t)GEN_TILE * S * G;
  auto kern = encode_generic_kernel<D, DSUB>;
  hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                                     (int)lds);
  if (e != hipSuccess) return e;
  kern<<<dim3((unsigned)(tiles * n_books)), dim3(256), lds, st>>>(
      x, xt, cb, codes, n_seq, seq_stride, n_rows, code_stride, code_row0, tiles, S, C,
      pre_rotated, sm.f, sm.n_scale);
  return hipGetLastError();
}

hipError_t launch_encode(const void* x, int xt, int D, int G, int S, int C, int64_t n_books,
                         int64_t n_seq, int64_t seq_stride, int64_t n_rows, const float* cb,
                         uint8_t* codes, int64_t code_stride, int64_t code_row0, int pre_rotated,
                         int force_generic, int packed_in_ws, void* ws, Smooth sm,
                         hipStream_t st) {
  if (n_books == 0 || n_seq == 0 || n_rows == 0) return hipSuccess;
  if (!force_generic && encode_mfma_eligible(D, G, S, C, xt)) {
    uint8_t* packed = reinterpret_cast<uint8_t*>(ws);
    if (!packed_in_ws) {
      const int64_t n_pack = n_books * S * G * 256;
      int64_t pblocks = (n_pack + 255) / 256;
      if (pblocks > 4096) pblocks = 4096;
      pack_codebooks_kernel<<<dim3((unsigned)pblocks), dim3(256), 0, st>>>(cb, packed, n_books, S,
                                                                         G);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
#define KVQ_MF(SS)                                                                          \
  if (S == SS) {                                                                           \
    if (xt == 1) return launch_mfma_t<SS, 1>(x, packed, codes, n_books, n_seq, seq_stride,  \
                                             n_rows, code_stride, code_row0, pre_rotated,   \
                                             sm, st);                                       \
    return launch_mfma_t<SS, 2>(x, packed, codes, n_books, n_seq, seq_stride, n_rows,       \
                                code_stride, code_row0, pre_rotated, sm, st);               \
  }
    KVQ_MF(1) KVQ_MF(2) KVQ_MF(3) KVQ_MF(4)
#undef KVQ_MF
  }
  const int dsub = D / G;
#define KVQ_GEN(DD, DS) \
  if (D == DD && dsub == DS) \
    return launch_generic_t<DD, DS>(x, xt, cb, codes, n_books, n_seq, seq_stride, n_rows,      \
                                    code_stride, code_row0, S, C, pre_rotated, sm, st);
  KVQ_GEN(64, 8) KVQ_GEN(64, 16) KVQ_GEN(64, 32) KVQ_GEN(64, 64)
  KVQ_GEN(128, 8) KVQ_GEN(128, 16) KVQ_GEN(128, 32) KVQ_GEN(128, 64) KVQ_GEN(128, 128)
  KVQ_GEN(256, 8) KVQ_GEN(256, 16) KVQ_GEN(256, 32) KVQ_GEN(256, 64) KVQ_GEN(256, 128)
#undef KVQ_GEN
  return hipErrorInvalidValue;
}

}  // namespace kvq
