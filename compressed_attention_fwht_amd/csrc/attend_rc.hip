// Decode attention over uint8 codes for the common cache shapes -- head_dim
// 128, C = 256 codewords, code rows of 32 or 64 bytes: 2 or 4 stages of 16
// groups of 8 dims, or 1 or 2 stages of 32 groups of 4 dims -- with LDS
// tables laid out so that code-driven gathers and histogram atomics never
// collide on a bank.
//
// What is computed is the same as in attend.hip: the query is rotated once
// and the inverse rotation of the keys absorbed into it ("VeloxQuant-MLX
// 0.5.1", VecInfer); keys are scored in the compressed domain through a
// per-query table ("Differential-KV" README, Decode & Prefill Innovations);
// values are accumulated as a per-(stage, group) histogram of softmax
// weights and contracted with the codebook once per chunk; each split-K chunk
// and each block of the fp16 window emits an fp32 partial (m, l, o_rot) that
// attn_merge_kernel combines by log-sum-exp and unrotates ("Differential-KV"
// README, Flash-Style LSE Combine; "VQKV" summary, 3. Inference Integration).
//
// The layout.  Per (token, stage, group) the K side reads one table entry
// (the four query heads' q_rot . c, 16 bytes) and the V side adds the token's
// fixed-point weights into one bin (two 64-bit words, two heads' 32-bit
// fields each).  Both are picked by a random code byte c.  gfx950 serves
// ds_read_b128, ds_read_b64 and ds_add_u64 sixteen lanes at a time and runs
// them at full rate when those sixteen lanes use different slots of a
// 256-byte bank row, whatever the rows are (measured: 13.7 lanes per cycle
// per CU for such b128 reads against 5.8 for random slots; 9.9 against 6.2
// for u64 atomics).  So a table row c holds the entries of 16 (stage,
// group) pairs in 16 slots, and each lane visits the pairs of its own token
// in an order rotated by its place p in its quarter wave: at every step the
// 16 lanes of a quarter sit on 16 different slots, for any codes.
//
// Geometry.  A code row (S*G bytes, [stage][group]) is cut into segments of
// 32 bytes (two stages of 16 groups, or one of 32); one segment's table lives
// in LDS at a time: LUT entries [region][c][slot] of 16 bytes, histogram bins
// [region][c][pair][slot] of 8 bytes, a region being 64 KiB (c at bits 8-15 of
// the LDS address).  A segment is two units of 16 bytes (4 dwords); the byte
// e = 16u + 4d + i of a segment (unit u, dword d, byte i) sits in region
// d >> 1, slot 8u + 4(d & 1) + i.  (One-stage caches of 16 groups, whose
// 16-byte rows would fill one region only, run faster on attend.hip's kernel
// and are not routed here.)
//
// The rotation moves no data.  Lane p loads unit (kc ^ p0) into unit slot kc
// (p0 = p & 1: the address does it); for step (kc, jj, q) a first
// v_perm_b32 takes dword 2jj + (q ^ p1) of the unit (p1 = bit 1 of p) with
// its bytes in the order i ^ (p >> 2); a second v_perm_b32 per code writes
// the code byte into bits 8-15 of the LDS address next to the slot offset
// (from a per-lane constant) and the region byte jj.  That is 1.25 VALU
// instructions per code for the address, and the slot of lane p at step
// (kc, jj, q, i) is 8(kc ^ p0) + 4(q ^ p1) + (i ^ p >> 2): sixteen values for
// the sixteen p (checked exhaustively on the host when the scheme was
// designed).
//
// Block: 1024 threads, one (sequence, KV head, four query heads) unit and a
// chunk of at most 4096 tokens, RC_TPT per thread (token t0 + tid + 1024 k),
// code rows held in registers.  K: per segment, the LUT segment staged from
// attn_rc_prep_kernel's output, gathers summed per token.  Chunk max and
// weight sum per head; the weights as fixed-point integers with F = 31 -
// ceil(log2 l) fraction bits (at most chunk * 2^-32 of the chunk's mass moved
// by rounding); tokens whose four weights round to zero add nothing and are
// skipped.  V: per segment, the histogram cleared, ds_add_u64 per code and
// head pair, then the contraction o_rot += 2^-F sum_c W[c] C^V[c] over the
// segment's stages, each thread keeping one group's 8 (or 4) dims for 4 heads.
#include "attend_common.h"

namespace kvq {

constexpr int RC_THREADS = 1024;
constexpr int RC_TPT = RC_MAX_CHUNK / RC_THREADS;
constexpr int RC_PF = 2;           // tokens of a lane whose code loads run ahead of its work
                                   // (1 with four stages, for registers)
// window tokens per window block: one row pass of the 512-thread block (32
// rows of 16 lanes), so its loads are a single round trip
constexpr int RC_WIN_BLOCK = 32;
// window tokens a chunk block takes into its own record at most (rows of
// its first 8 waves); a longer share goes to window blocks
constexpr int RC_WIN_SLICE = 32;

// The chunk kernel declares no static LDS, so its dynamic LDS (the table)
// starts at LDS address 0 and a perm-built table offset is the address
// itself: these accessors take it as an absolute LDS address (a pointer
// derived from the extern array would add the array's address as a separate
// instruction, its value being fixed only after code generation).
typedef __attribute__((address_space(3))) f32x4_t lds_f32x4;
typedef __attribute__((address_space(3))) unsigned long long lds_u64;
__device__ __forceinline__ f32x4_t lds_read128(uint32_t a) {
  return *(const lds_f32x4*)(a);
}
__device__ __forceinline__ void lds_add64(uint32_t a, unsigned long long v) {
  __hip_atomic_fetch_add((lds_u64*)(a), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// Barrier for LDS data only: this wave's LDS operations complete, then the
// workgroup meets.  __syncthreads() also drains every outstanding global
// load first, which would expose the latency of the code rows this kernel
// keeps in flight across its phases; the LDS-DMA table copies are waited for
// explicitly (vmcnt) where they are needed.  The memory clobber keeps the
// compiler from moving memory accesses across it.
__device__ __forceinline__ void lds_sync() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

template <int SG>
struct RcGeom {
  static_assert(SG == 32 || SG == 64, "two or four stages of 16 groups");
  static constexpr int NSEG = SG / 32;                  // table segments per row
  static constexpr int SEGB = 32;                       // code bytes per segment
  static constexpr int UNITB = SEGB / 2;                // bytes per unit
  static constexpr int UDW = UNITB / 4;                 // dwords per unit
  static constexpr int TAB = 131072;                    // LDS table bytes per segment
  static constexpr int NPART = 32;                      // contraction partials per group
};

// Region and slot of segment byte e.
__host__ __device__ constexpr int rc_region(int e) { return ((e >> 2) & 3) >> 1; }
__host__ __device__ constexpr int rc_slot(int e) {
  return 8 * (e >> 4) + 4 * ((e >> 2) & 1) + (e & 3);
}

// --------------------------------------------------------- attn_rc_prep
// grid: n_lb LUT blocks, SG/2 codebook blocks, units * n_wb window blocks;
// 512 threads.  A LUT block writes one quarter of the codewords (64) of one
// table region (16 slots) of one segment of one unit: scale * H q / sqrt(D)
// for the unit's four heads (heads past the group's last repeat it; never
// read back) dotted with C^K_sg[c], sixteen consecutive threads writing the
// sixteen slots of a codeword's 256-byte row.  A codebook block copies V
// codebook rows into the order the chunk kernel's contraction reads them,
// cvt[segment][c][region][slot][8], so that the sixteen lanes of a quarter
// wave, on the sixteen slots of one region and one codeword, read 512
// contiguous bytes.  A window block computes the softmax partial of up to
// RC_WIN_BLOCK window tokens (record n_chunks + block of the unit's heads).
template <int SG, int NG>
__global__ __launch_bounds__(512) void attn_rc_prep_kernel(
    const float* __restrict__ q, const float* __restrict__ kcb, const float* __restrict__ vcb,
    uint8_t* __restrict__ lut, float* __restrict__ cvt, float* __restrict__ part,
    const uint16_t* __restrict__ kw, const uint16_t* __restrict__ vw, int B, int Hq, int Hkv,
    int n_hsplit, int n_wb, int W, int wstride, int n_chunks, int nslots, int pstride,
    float scale, const float* __restrict__ ksm, int64_t ksm_rows) {
  using Gm = RcGeom<SG>;
  constexpr int D = 128, L = 16, DS = D / NG;
  constexpr int NREG = 2;
  constexpr int LB_PER_UNIT = Gm::NSEG * NREG * 4;      // (segment, region, codeword quarter)
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  __shared__ float qs[4][D];
  const int units = B * Hkv * n_hsplit;
  const int nlb = units * LB_PER_UNIT;
  const int R = Hq / Hkv;
  const int tid = threadIdx.x, lane = tid & 63;
  int bid = blockIdx.x;
  if (bid >= nlb && bid < nlb + SG / 2) {               // V codebook -> contraction order
    const int row = (bid - nlb) * 512 + tid;             // (sg, c), one DS-float row each
    const int sg = row >> 8, c = row & 255;
    const int seg = sg >> 5, e = sg & 31;
    const float4* src = reinterpret_cast<const float4*>(vcb + (int64_t)row * DS);
    float4* dst = reinterpret_cast<float4*>(
        cvt + ((((int64_t)seg * 256 + c) * NREG + rc_region(e)) * 16 + rc_slot(e)) * DS);
#pragma unroll
    for (int i = 0; i < DS / 4; ++i) dst[i] = src[i];
    return;
  }
  const bool win = bid >= nlb;
  if (win) bid -= nlb + SG / 2;
  const int unit = win ? bid / n_wb : bid / LB_PER_UNIT;
  const int b = unit / (Hkv * n_hsplit);
  const int kvh = unit - b * (Hkv * n_hsplit);
  const int kv = kvh / n_hsplit, hs = kvh - kv * n_hsplit;
  const int h0 = kv * R + hs * 4;
  const int nh = (R - hs * 4) < 4 ? (R - hs * 4) : 4;
  if (win) {
    const int wb = bid - unit * n_wb;
    const int w0 = wb * RC_WIN_BLOCK;
    const int w1 = (w0 + RC_WIN_BLOCK) < W ? (w0 + RC_WIN_BLOCK) : W;
    window_partial<4, D, RC_WIN_BLOCK>(q, kw, vw, part, smem, b, kv, h0, nh, Hq, Hkv, wstride,
                                       w0, w1, n_chunks + wb, nslots, pstride, scale);
    return;
  }
  const int lb = bid - unit * LB_PER_UNIT;
  const int cq = lb & 3, region = (lb >> 2) % NREG, seg = (lb >> 2) / NREG;
  const int slot = tid & 15;
  // the segment byte e of (region, slot): inverse of rc_region / rc_slot
  const int u = slot >> 3, i = slot & 3;
  const int e = 16 * u + 4 * (2 * region + ((slot >> 2) & 1)) + i;
  const int sg = seg * 32 + e;
  const int g = sg % NG;
  // codebook rows first: their loads are in flight across the query rotation
  float cv[2][DS];
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int c = cq * 64 + (tid >> 4) + 32 * k;
    const float4* cp = reinterpret_cast<const float4*>(kcb + ((int64_t)sg * 256 + c) * DS);
#pragma unroll
    for (int i = 0; i < DS / 4; ++i) {
      const float4 c4 = cp[i];
      cv[k][4 * i] = c4.x; cv[k][4 * i + 1] = c4.y; cv[k][4 * i + 2] = c4.z; cv[k][4 * i + 3] = c4.w;
    }
  }
  if (tid < 64) {                                       // wave 0: the four query rows
    const int r = lane / L;
    const int h = h0 + (r < nh ? r : nh - 1);
    const float4* qp = reinterpret_cast<const float4*>(q + ((int64_t)b * Hq + h) * D + (lane % L) * 8);
    const float4 x0 = qp[0], x1 = qp[1];
    float v[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
    if (ksm != nullptr) smooth_query<D>(v, ksm, b, kv, Hkv, ksm_rows, lane % L);
    hadamard_row<8, L>(v, lane);
    const float rs = scale * rsqrt_pow2(D);
#pragma unroll
    for (int e2 = 0; e2 < 8; ++e2) qs[r][(lane % L) * 8 + e2] = v[e2] * rs;
  }
  __syncthreads();
  float qv[4][DS];
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int j = 0; j < DS; ++j) qv[r][j] = qs[r][g * DS + j];
  uint8_t* dst = lut + (size_t)unit * (Gm::NSEG * Gm::TAB) + (size_t)seg * Gm::TAB +
                 (size_t)region * 65536 + slot * 16;
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int c = cq * 64 + (tid >> 4) + 32 * k;
    float acc[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      acc[r] = 0.0f;
#pragma unroll
      for (int j = 0; j < DS; ++j) acc[r] = __builtin_fmaf(qv[r][j], cv[k][j], acc[r]);
    }
    *reinterpret_cast<float4*>(dst + c * 256) = make_float4(acc[0], acc[1], acc[2], acc[3]);
  }
}

// ------------------------------------------------------------- attn_rc
// grid (n_chunks, Hkv * n_hsplit, B), RC_THREADS threads, Gm::TAB bytes of
// dynamic LDS for one table segment (the contraction's partials reuse it)
// plus the block reductions.
template <int SG, int NG>
__global__ __launch_bounds__(RC_THREADS, 1) void attn_rc_kernel(
    const uint8_t* __restrict__ kcodes, const uint8_t* __restrict__ vcodes,
    const float* __restrict__ cvt, const uint8_t* __restrict__ lut, float* __restrict__ part,
    int Hq, int Hkv, int n_hsplit, int Tc, int chunk, int nslots, int pstride, int cstride,
    const float* __restrict__ q, const uint16_t* __restrict__ kw,
    const uint16_t* __restrict__ vw, int W, int wslice, int wstride, float scale) {
  using Gm = RcGeom<SG>;
  constexpr int NSEG = Gm::NSEG, UDW = Gm::UDW, NW = RC_THREADS / 64;
  // dynamic LDS only, so the table starts at address 0 and a perm-built
  // address needs no base added: [0, TAB) table, then the reductions
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  float (*red_m)[4] = reinterpret_cast<float (*)[4]>(smem + Gm::TAB);
  float (*red_l)[4] = reinterpret_cast<float (*)[4]>(smem + Gm::TAB + NW * 16);
  uint32_t (*red_w)[4] = reinterpret_cast<uint32_t (*)[4]>(smem + Gm::TAB + 2 * NW * 16);

  // Workgroups are handed to the eight XCDs round-robin by linear id; the
  // ids are renumbered so that each XCD runs whole units (all chunks of a
  // few (sequence, KV head) pairs), so its L2 holds those units' tables only.
  int ci, unit, b;
  {
    const int nx = gridDim.x, ny = gridDim.y, nb = nx * ny * gridDim.z;
    int lin = blockIdx.x + nx * (blockIdx.y + ny * blockIdx.z);
    if ((nb & 7) == 0) lin = (lin & 7) * (nb >> 3) + (lin >> 3);
    ci = lin % nx;
    const int rest = lin / nx;
    unit = rest % ny;
    b = rest / ny;
  }
  const int kv = unit / n_hsplit, hs = unit - kv * n_hsplit;
  const int R = Hq / Hkv;
  const int h0 = kv * R + hs * 4;
  const int nh = (R - hs * 4) < 4 ? (R - hs * 4) : 4;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint32_t p = lane & 15, p0 = p & 1, p1 = (p >> 1) & 1, p2 = (p >> 2) & 1, p3 = p >> 3;
  const uint32_t p23 = p >> 2;
  const int t0 = ci * chunk;
  const int t1 = (t0 + chunk) < Tc ? (t0 + chunk) : Tc;
  const int64_t rowbase = ((int64_t)b * Hkv + kv) * (int64_t)cstride;
  const uint8_t* lsrc = lut + ((size_t)b * Hkv * n_hsplit + unit) * (size_t)(NSEG * Gm::TAB);

  // ---- window slice: tokens [ci * wslice, ...) of the unit's dense fp16
  // window (at most RC_WIN_SLICE), one per row of 16 lanes (8 dims each).
  // Its loads go out first; its softmax partial (own max, float weights, V
  // rotated like the codebooks) is formed around the first LUT staging and
  // kept in LDS, and folded into the chunk's record at the end.
  float (*wred_m)[4] = reinterpret_cast<float (*)[4]>(smem + Gm::TAB + 3 * NW * 16);
  float (*wred_l)[4] = reinterpret_cast<float (*)[4]>(smem + Gm::TAB + 4 * NW * 16);
  float* wpart = reinterpret_cast<float*>(smem + Gm::TAB + 5 * NW * 16);  // [8][4][128]
  const int wa = ci * wslice < W ? ci * wslice : W;
  const int nwin = ((wa + wslice) < W ? (wa + wslice) : W) - wa;   // block-uniform
  const int wrow = tid >> 4, wcol = tid & 15;
  const bool wact = wrow < nwin;
  const int nww = (nwin + 3) >> 2;                      // waves holding window rows
  const bool wwave = wave < nww;                        // wave-uniform
  uint4 kraw = make_uint4(0u, 0u, 0u, 0u), vraw = kraw;
  float qv[4][8], sw[4];
  if (wwave) {
    const int64_t off = (((int64_t)b * Hkv + kv) * wstride + wa + (wact ? wrow : 0)) * 128 + wcol * 8;
    kraw = *reinterpret_cast<const uint4*>(kw + off);
    vraw = *reinterpret_cast<const uint4*>(vw + off);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float4* qp = reinterpret_cast<const float4*>(
          q + ((int64_t)b * Hq + h0 + (r < nh ? r : nh - 1)) * 128 + wcol * 8);
      const float4 x0 = qp[0], x1 = qp[1];
      qv[r][0] = x0.x; qv[r][1] = x0.y; qv[r][2] = x0.z; qv[r][3] = x0.w;
      qv[r][4] = x1.x; qv[r][5] = x1.y; qv[r][6] = x1.z; qv[r][7] = x1.w;
    }
  }

  // ---- per-lane constants of the rotation (see the file comment): SE[q]
  // picks dword 2jj + (q ^ p1) of a pair with its bytes in the order
  // i ^ (p >> 2); LK / LV hold the two slot offsets (16- and 8-byte
  // entries) of the lane's step (unit slot kc, q, i >> 1) and the region
  // bytes 0 and 1; SA[i][jj] picks the slot offset by bit 0 of i ^ (p >> 2),
  // the code byte i, and region jj.
  constexpr int NJ = UDW / 2;                           // dword pairs per unit
  uint32_t SE[2], SA[4][NJ];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    SE[q] = 0u;
#pragma unroll
    for (int i = 0; i < 4; ++i) SE[q] |= (4u * ((uint32_t)q ^ p1) + ((uint32_t)i ^ p23)) << (8 * i);
  }
#pragma unroll
  for (int jj = 0; jj < NJ; ++jj)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      SA[i][jj] = (((uint32_t)i & 1u) ^ p2) | ((4u + (uint32_t)i) << 8) |
                  ((2u + (uint32_t)jj) << 16) | (12u << 24);
  // slot-offset constants with entry size ES (16 for the LUT, 8 for the
  // histogram), built where each pass starts
  auto slot_consts = [&](uint32_t (&L)[2][2][2], uint32_t es) {
#pragma unroll
    for (int q = 0; q < 2; ++q)
#pragma unroll
      for (int kc = 0; kc < 2; ++kc)
#pragma unroll
        for (int i1 = 0; i1 < 2; ++i1) {
          const uint32_t base =
              8u * ((uint32_t)kc ^ p0) + 4u * ((uint32_t)q ^ p1) + 2u * ((uint32_t)i1 ^ p3);
          L[kc][q][i1] = (base * es) | ((base + 1u) * es << 8) | (1u << 24);
        }
  };

  // ---- code rows streamed per segment: a ring of RC_PF + 1 buffers holds
  // the segment's bytes of the lane's current token and of the next RC_PF
  // ones, units in the lane's rotated order.  A segment's bytes are half a
  // row (two segments) or all of it; the second segment's half-rows come
  // from the caches, the first pass having brought the whole lines in.
  constexpr int PF = SG == 64 ? 1 : RC_PF, NB = PF + 1;
  uint32_t RB[NB][2][UDW];
  auto load_seg = [&](const uint8_t* __restrict__ codes, int k, int seg, uint32_t (&dst)[2][UDW]) {
    const int t = t0 + tid + RC_THREADS * k;
    const int tl = t < t1 ? t : t1 - 1;
    const uint8_t* row = codes + (rowbase + tl) * SG + seg * Gm::SEGB;
#pragma unroll
    for (int kc = 0; kc < 2; ++kc) {
      const uint8_t* src = row + ((uint32_t)kc ^ p0) * Gm::UNITB;
      const uint4 v = *reinterpret_cast<const uint4*>(src);
      dst[kc][0] = v.x; dst[kc][1] = v.y; dst[kc][2] = v.z; dst[kc][3] = v.w;
    }
  };
  // code bytes of (unit slot kc, pair jj, member q) in visiting order
  auto codes4 = [&](const uint32_t (&w)[2][UDW], int kc, int jj, int q) -> uint32_t {
    return __builtin_amdgcn_perm(w[kc][2 * jj + 1], w[kc][2 * jj], SE[q]);
  };
  auto stage = [&](int seg) {                           // LUT segment -> LDS, 1 KiB per wave step
    const uint8_t* src = lsrc + (size_t)seg * Gm::TAB;
#pragma unroll
    for (int piece = wave; piece < Gm::TAB / 1024; piece += NW)
      __builtin_amdgcn_global_load_lds(src + piece * 1024 + lane * 16,
                                       (__attribute__((address_space(3))) void*)(smem + piece * 1024),
                                       16, 0, 0);
  };
  // the first PF tokens' loads of a pass, issued after anything whose
  // completion the pass waits for explicitly (vector loads complete in order)
  auto prime = [&](const uint8_t* __restrict__ codes, int seg) {
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int k = 0; k < PF && k < RC_TPT; ++k) load_seg(codes, k, seg, RB[k]);
    __builtin_amdgcn_sched_barrier(0);
  };

  // ---- K: scores from the LUT
  uint32_t LK[2][2][2];
  slot_consts(LK, 16u);
  float acc[RC_TPT][4];
#pragma unroll
  for (int k = 0; k < RC_TPT; ++k)
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[k][r] = 0.0f;
#pragma unroll
  for (int seg = 0; seg < NSEG; ++seg) {
    if (seg > 0) lds_sync();                       // every read of the previous segment done
    stage(seg);
    prime(kcodes, seg);
    __builtin_amdgcn_s_waitcnt(0x0f70);                 // vmcnt(0): the LUT segment has landed
                                                        // (with the first rows, in flight with it)
    if (seg == 0 && wwave) {                            // window scores, wave maxima
      const uint32_t kr[4] = {kraw.x, kraw.y, kraw.z, kraw.w};
      float kx[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        kx[2 * i] = f16_bits_to_f32(kr[i]);
        kx[2 * i + 1] = f16_bits_to_f32(kr[i] >> 16);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float dot = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) dot = __builtin_fmaf(qv[r][e], kx[e], dot);
        dot = row_sum<16>(dot) * scale;
        sw[r] = wact ? dot : -__builtin_inff();
        const float mw = wave_max(sw[r]);
        if (lane == 0) wred_m[wave][r] = mw;
      }
    }
    lds_sync();
    if (seg == 0 && wwave) {                            // window weights, p * H v / sqrt(D)
      const uint32_t vr[4] = {vraw.x, vraw.y, vraw.z, vraw.w};
      float vx[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        vx[2 * i] = f16_bits_to_f32(vr[i]);
        vx[2 * i + 1] = f16_bits_to_f32(vr[i] >> 16);
      }
      hadamard_row<8, 16>(vx, lane);
#pragma unroll
      for (int e = 0; e < 8; ++e) vx[e] *= rsqrt_pow2(128);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float mw = wred_m[0][r];
        for (int w = 1; w < nww; ++w) mw = fmaxf(mw, wred_m[w][r]);
        const float pf = wact ? __expf(sw[r] - mw) : 0.0f;
        const float lw = wave_sum(wcol == 0 ? pf : 0.0f);
        if (lane == 0) wred_l[wave][r] = lw;
#pragma unroll
        for (int e = 0; e < 8; ++e) {                   // the wave's 4 rows summed
          float a = pf * vx[e];
          a = pair_sum<16>(a);
          a = pair_sum<32>(a);
          if (lane < 16) wpart[(wave * 4 + r) * 128 + wcol * 8 + e] = a;
        }
      }
    }
#pragma unroll
    for (int k = 0; k < RC_TPT; ++k) {
      if (k + PF < RC_TPT) load_seg(kcodes, k + PF, seg, RB[(k + PF) % NB]);
#pragma unroll
      for (int kc = 0; kc < 2; ++kc)
#pragma unroll
        for (int jj = 0; jj < NJ; ++jj)
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const uint32_t e4 = codes4(RB[k % NB], kc, jj, q);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const uint32_t a = __builtin_amdgcn_perm(e4, LK[kc][q][i >> 1], SA[i][jj]);
            const f32x4_t v = lds_read128(a);
            acc[k][0] += v[0]; acc[k][1] += v[1]; acc[k][2] += v[2]; acc[k][3] += v[3];
            // the sums are formed here, not deferred past the next gathers
            asm volatile("" : "+v"(acc[k][0]), "+v"(acc[k][1]), "+v"(acc[k][2]), "+v"(acc[k][3]));
          }
          // keep the scheduler from hoisting every gather of the thread ahead
          // of its sums: 4 in flight per wave here, 16 waves per CU
          __builtin_amdgcn_sched_barrier(0);
        }
    }
  }

  // ---- chunk max, weights, weight sum per head
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    float v = -__builtin_inff();
#pragma unroll
    for (int k = 0; k < RC_TPT; ++k) {
      const bool ok = t0 + tid + RC_THREADS * k < t1;
      acc[k][r] = ok ? acc[k][r] : -__builtin_inff();
      v = fmaxf(v, acc[k][r]);
    }
    v = wave_max(v);
    if (lane == 0) red_m[wave][r] = v;
  }
  lds_sync();                                      // also: every LUT read is done
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    float v = red_m[0][r];
#pragma unroll
    for (int w = 1; w < NW; ++w) v = fmaxf(v, red_m[w][r]);
    float sp = 0.0f;
#pragma unroll
    for (int k = 0; k < RC_TPT; ++k) {
      acc[k][r] = __expf(acc[k][r] - v);                // -inf (no token) -> 0
      sp += acc[k][r];
    }
    sp = wave_sum(sp);
    if (lane == 0) red_l[wave][r] = sp;
  }
  auto clear = [&]() {
#pragma unroll
    for (int i = tid; i < Gm::TAB / 16; i += RC_THREADS)
      reinterpret_cast<uint4*>(smem)[i] = make_uint4(0u, 0u, 0u, 0u);
  };
  clear();
  lds_sync();                                      // red_l complete
  // fraction bits of head r, from the chunk's weight sum (the same sum in
  // every thread, so every thread derives the same F)
  auto frac_scale = [&](int r) -> float {
    float l = red_l[0][r];
#pragma unroll
    for (int w = 1; w < NW; ++w) l += red_l[w][r];
    return (float)(1u << (31 - ceil_log2_f(l)));
  };
  uint64_t W0[RC_TPT], W1[RC_TPT];
  {
    float fsc[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) fsc[r] = frac_scale(r);
    uint32_t ws[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int k = 0; k < RC_TPT; ++k) {
      uint32_t w[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        w[r] = (uint32_t)__builtin_rintf(acc[k][r] * fsc[r]);
        ws[r] += w[r];
      }
      W0[k] = (uint64_t)w[0] | ((uint64_t)w[1] << 32);
      W1[k] = (uint64_t)w[2] | ((uint64_t)w[3] << 32);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const uint32_t v = wave_sum_u32(ws[r]);
      if (lane == 0) red_w[wave][r] = v;
    }
  }

  // ---- V: histogram per segment, then its share of the contraction
  // contraction mapping: quarter Q = tid / 16 reads slot p of region (Q & 1)
  // for its range of codewords; the slot names the segment byte e and so its
  // (stage, group): with 16 groups of 8 dims a segment holds two stages (bytes
  // e and e + 16 are one group, lanes p and p ^ 8), with 32 groups of 4 dims
  // one stage (byte e is group e).  The group is the same in every segment.
  constexpr int DS = 128 / NG;
  const int Q = tid >> 4;
  const int creg = Q & 1, cn = 8, c0 = (Q >> 1) * 8;
  const int grp = 4 * (2 * creg + (int)((p >> 2) & 1)) + (int)(p & 3) +
                  (NG == 16 ? 0 : 16 * (int)(p >> 3));   // the segment byte's group
  uint32_t LV[2][2][2];
  slot_consts(LV, 8u);
  float o[4][DS];
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int j = 0; j < DS; ++j) o[r][j] = 0.0f;
#pragma unroll
  for (int seg = 0; seg < NSEG; ++seg) {
    if (seg > 0) {
      lds_sync();                                  // contraction reads of the last segment done
      clear();
    }
    prime(vcodes, seg);
    lds_sync();                                    // the histogram is clear
#pragma unroll
    for (int k = 0; k < RC_TPT; ++k) {
      if (k + PF < RC_TPT) load_seg(vcodes, k + PF, seg, RB[(k + PF) % NB]);
      // the token's code bytes in visiting order, formed (and marked used)
      // ahead of the skip test: with its first use inside the branch the
      // compiler sinks the row's load (a read-only argument, so no barrier
      // orders it) past the barrier into the branch
      uint32_t e4s[2][NJ][2];
#pragma unroll
      for (int kc = 0; kc < 2; ++kc)
#pragma unroll
        for (int jj = 0; jj < NJ; ++jj)
#pragma unroll
          for (int q = 0; q < 2; ++q) {
            e4s[kc][jj][q] = codes4(RB[k % NB], kc, jj, q);
            asm volatile("" ::"v"(e4s[kc][jj][q]));
          }
      if ((W0[k] | W1[k]) != 0ull) {
#pragma unroll
        for (int kc = 0; kc < 2; ++kc)
#pragma unroll
          for (int jj = 0; jj < NJ; ++jj)
#pragma unroll
          for (int q = 0; q < 2; ++q) {
            const uint32_t e4 = e4s[kc][jj][q];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const uint32_t a = __builtin_amdgcn_perm(e4, LV[kc][q][i >> 1], SA[i][jj]);
              lds_add64(a, W0[k]);
              lds_add64(a + 128, W1[k]);
            }
            __builtin_amdgcn_sched_barrier(0);
          }
      }
    }
    lds_sync();
    // this lane's rows: histogram bins (region creg, slot p) and codebook
    // rows of its (stage, group), codewords c0 .. c0 + cn - 1, one codeword
    // ahead in flight (a rolled loop, so registers stay bounded)
    constexpr int NREG = 2;
    const uint8_t* hp = smem + creg * 65536 + c0 * 256 + p * 8;
    const float4* cp = reinterpret_cast<const float4*>(
        cvt + ((((int64_t)seg * 256 + c0) * NREG + creg) * 16 + p) * DS);
    constexpr int CSTEP = NREG * 16 * DS / 4;           // float4s from one codeword to the next
    constexpr int NX = DS / 4;                          // float4s of one codebook row
    uint2 wa = *reinterpret_cast<const uint2*>(hp), wb = *reinterpret_cast<const uint2*>(hp + 128);
    float4 x[NX];
#pragma unroll
    for (int i = 0; i < NX; ++i) x[i] = cp[i];
#pragma unroll 1
    for (int cc = 0; cc < cn; ++cc) {
      const uint2 na = *reinterpret_cast<const uint2*>(hp + 256 * (cc + 1 < cn ? cc + 1 : cc));
      const uint2 nb = *reinterpret_cast<const uint2*>(hp + 128 + 256 * (cc + 1 < cn ? cc + 1 : cc));
      const float4* np = cp + CSTEP * (cc + 1 < cn ? cc + 1 : cc);
      float4 nx[NX];
#pragma unroll
      for (int i = 0; i < NX; ++i) nx[i] = np[i];
      const float wf[4] = {(float)wa.x, (float)wa.y, (float)wb.x, (float)wb.y};
      float cv[DS];
#pragma unroll
      for (int i = 0; i < NX; ++i) {
        cv[4 * i] = x[i].x; cv[4 * i + 1] = x[i].y; cv[4 * i + 2] = x[i].z; cv[4 * i + 3] = x[i].w;
      }
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int j = 0; j < DS; ++j) o[r][j] = __builtin_fmaf(wf[r], cv[j], o[r][j]);
      wa = na; wb = nb;
#pragma unroll
      for (int i = 0; i < NX; ++i) x[i] = nx[i];
    }
  }
  // ---- partials of one group: lanes sharing it summed by lane exchanges,
  // then across waves / quarters through LDS (the table is free now)
  if constexpr (NG == 16) {
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int j = 0; j < DS; ++j) {
        o[r][j] += xor_lane<8>(o[r][j]);                // the two stages of the segment pair
      }
  }
  lds_sync();
  float* buf = reinterpret_cast<float*>(smem);          // [NPART][4][128]
  const bool writer = NG == 16 ? (p & 8) == 0 : true;
  const int pi = Q >> 1;
  if (writer) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float4* dp = reinterpret_cast<float4*>(buf + (pi * 4 + r) * 128 + grp * DS);
#pragma unroll
      for (int i = 0; i < DS / 4; ++i)
        dp[i] = make_float4(o[r][4 * i], o[r][4 * i + 1], o[r][4 * i + 2], o[r][4 * i + 3]);
    }
  }
  lds_sync();
  if (tid < 512) {
    const int r = tid >> 7, d = tid & 127;
    float v = 0.0f;
#pragma unroll 8
    for (int i = 0; i < Gm::NPART; ++i) v += buf[(i * 4 + r) * 128 + d];
    const float inv = 1.0f / frac_scale(r);
    float mm = red_m[0][r];
    for (int w = 1; w < NW; ++w) mm = fmaxf(mm, red_m[w][r]);
    if (r < nh) {
      uint32_t li = 0u;
      for (int w = 0; w < NW; ++w) li += red_w[w][r];
      float l = (float)li * inv;
      v *= inv;
      if (nwin > 0) {                                   // fold the window slice in
        float mw = wred_m[0][r], lw = 0.0f, ow = 0.0f;
        for (int w = 1; w < nww; ++w) mw = fmaxf(mw, wred_m[w][r]);
        for (int w = 0; w < nww; ++w) {
          lw += wred_l[w][r];
          ow += wpart[(w * 4 + r) * 128 + d];
        }
        const float M = fmaxf(mm, mw);
        const float a = __expf(mm - M), aw = __expf(mw - M);
        v = v * a + ow * aw;
        l = l * a + lw * aw;
        mm = M;
      }
      float* pp = part + ((int64_t)(b * Hq + h0 + r) * nslots + ci) * pstride;
      pp[4 + d] = v;
      if (d == 0) {
        pp[0] = mm;
        pp[1] = l;
      }
    }
  }
}

// ------------------------------------------------------------- launcher
// Code rows of 32 or 64 bytes: two or four stages of 16 groups of 8 dims, or
// one or two stages of 32 groups of 4 dims (the product codebooks of 2-bit
// scalar codes).  One-stage caches of 16 groups are small (16 code bytes per
// token): their decode is bound by memory round trips and launches, which the
// general kernel, with its LUT built inside the chunk blocks and no separate
// LUT pass, keeps fewer of; they stay there.
bool attn_rc_eligible(int D, int G, int S, int C, int Hq, int Hkv, int Tc) {
  const bool rows = (G == 16 && (S == 2 || S == 4)) || (G == 32 && (S == 1 || S == 2));
  return D == 128 && C == 256 && rows && Tc > 0 && Hq / Hkv >= 2;
}

size_t attn_rc_table_bytes(int S, int G) { return (size_t)131072 * (S * G / 32); }

int attn_rc_window_slice(int W, int n_chunks) {
  const int per = n_chunks > 0 ? (W + n_chunks - 1) / n_chunks : 0;
  return per <= RC_WIN_SLICE ? per : 0;
}

int attn_rc_window_blocks(int W) { return (W + RC_WIN_BLOCK - 1) / RC_WIN_BLOCK; }

template <int SG, int NG>
static hipError_t launch_rc_sg(const AttnPlan& p, int B, int Hq, int Hkv, int Tc, int W,
                               int cstride, int wstride, float scale, const float* q,
                               const uint8_t* kc, const uint8_t* vc, const float* kcb,
                               const float* vcb, const uint16_t* kw, const uint16_t* vw,
                               uint8_t* lut, float* part, Smooth ksm, hipStream_t st) {
  using Gm = RcGeom<SG>;
  const int units = B * Hkv * p.n_hsplit;
  const int nslots = p.n_chunks + p.n_wblocks;
  const size_t wl = p.n_wblocks ? ((size_t)RC_WIN_BLOCK * 4 + (size_t)8 * 4 * 128) * 4 : 0;
  constexpr int LB_PER_UNIT = Gm::NSEG * 2 * 4;
  float* cvt = reinterpret_cast<float*>(lut + (size_t)units * p.lut_slice);
  hipError_t e;
  if (wl > 0) {
    e = hipFuncSetAttribute((const void*)attn_rc_prep_kernel<SG, NG>,
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)wl);
    if (e != hipSuccess) return e;
  }
  attn_rc_prep_kernel<SG, NG><<<dim3(units * LB_PER_UNIT + SG / 2 + units * p.n_wblocks), 512, wl,
                                st>>>(
      q, kcb, vcb, lut, cvt, part, kw, vw, B, Hq, Hkv, p.n_hsplit, p.n_wblocks, W, wstride,
      p.n_chunks, nslots, p.pstride, scale, ksm.f, ksm.n_scale);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  // table, block reductions, window maxima and sums, window partials
  const int lds = Gm::TAB + 5 * (RC_THREADS / 64) * 16 + RC_WIN_SLICE / 4 * 4 * 128 * 4;
  e = hipFuncSetAttribute((const void*)attn_rc_kernel<SG, NG>,
                          hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (e != hipSuccess) return e;
  attn_rc_kernel<SG, NG><<<dim3(p.n_chunks, Hkv * p.n_hsplit, B), RC_THREADS, lds, st>>>(
      kc, vc, cvt, lut, part, Hq, Hkv, p.n_hsplit, Tc, p.chunk, nslots, p.pstride, cstride, q, kw,
      vw, W, p.wslice, wstride, scale);
  return hipGetLastError();
}

hipError_t launch_attend_rc(const AttnPlan& p, int B, int Hq, int Hkv, int S, int G, int Tc,
                            int W, int cstride, int wstride, float scale, const float* q,
                            const uint8_t* kc, const uint8_t* vc, const float* kcb,
                            const float* vcb, const uint16_t* kw, const uint16_t* vw,
                            uint8_t* lut, float* part, Smooth ksm, hipStream_t st) {
#define KVQ_RC(SS, GG)                                                                        \
  if (S == SS && G == GG)                                                                     \
    return launch_rc_sg<SS * GG, GG>(p, B, Hq, Hkv, Tc, W, cstride, wstride, scale, q, kc, vc, \
                                     kcb, vcb, kw, vw, lut, part, ksm, st);
  KVQ_RC(2, 16) KVQ_RC(4, 16) KVQ_RC(1, 32) KVQ_RC(2, 32)
#undef KVQ_RC
  return hipErrorInvalidValue;                          // the plan routes no other here
}

}  // namespace kvq
