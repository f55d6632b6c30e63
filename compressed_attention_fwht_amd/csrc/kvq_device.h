// Device helpers shared by the gfx950 kernels of libkvq: element loads,
// bf16 packing, wavefront exchanges and the Walsh-Hadamard butterfly.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvq {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4_t;

// ---------------------------------------------------------------- elements
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float f16_bits_to_f32(uint32_t h) {
  return (float)__builtin_bit_cast(_Float16, (unsigned short)(h & 0xffffu));
}

// Round-to-nearest-even float -> bf16 bits (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16_rne(lo) | (f32_to_bf16_rne(hi) << 16);
}
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// Two floats -> packed bf16 pair (lo in bits 0-15), round to nearest even,
// by the hardware converter (v_cvt_pk_bf16_f32).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t cvt_pk_bf16(float lo, float hi) {
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// Load 8 consecutive elements of a row of type xt (0 f32, 1 bf16, 2 f16) as
// float.  p points at the first element; 16-byte aligned for bf16/f16, and
// 32-byte aligned rows for f32 are read as two 16-byte loads.
template <int XT>
__device__ __forceinline__ void load8(const void* p, float (&v)[8]) {
  if constexpr (XT == 0) {
    const float4* q = reinterpret_cast<const float4*>(p);
    float4 a = q[0], b = q[1];
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  } else {
    uint4 w = *reinterpret_cast<const uint4*>(p);
    uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if constexpr (XT == 1) {
        v[2 * i] = bf16_lo(ws[i]);
        v[2 * i + 1] = bf16_hi(ws[i]);
      } else {
        v[2 * i] = f16_bits_to_f32(ws[i]);
        v[2 * i + 1] = f16_bits_to_f32(ws[i] >> 16);
      }
    }
  }
}

// Four consecutive elements (16-byte aligned for f32, 8-byte for 2-byte types)
// as float32 into v[o..o+3].
template <int XT>
__device__ __forceinline__ void load4(const void* p, float (&v)[8], int o) {
  if constexpr (XT == 0) {
    const float4 a = *reinterpret_cast<const float4*>(p);
    v[o] = a.x; v[o + 1] = a.y; v[o + 2] = a.z; v[o + 3] = a.w;
  } else {
    const uint2 w = *reinterpret_cast<const uint2*>(p);
    const uint32_t ws[2] = {w.x, w.y};
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      if constexpr (XT == 1) {
        v[o + 2 * i] = bf16_lo(ws[i]);
        v[o + 2 * i + 1] = bf16_hi(ws[i]);
      } else {
        v[o + 2 * i] = f16_bits_to_f32(ws[i]);
        v[o + 2 * i + 1] = f16_bits_to_f32(ws[i] >> 16);
      }
    }
  }
}

// ------------------------------------------------------- lane exchanges
// Value of lane (lane ^ M) within the wavefront, for M in {1,2,4,8,16,32}.
// DPP or a permlane swap (VALU) where one instruction does it, ds_swizzle
// for M = 4.
template <int M>
__device__ __forceinline__ float xor_lane(float x) {
  int v = __float_as_int(x);
  int r;
  if constexpr (M == 1) {
    r = __builtin_amdgcn_mov_dpp(v, 0xB1, 0xF, 0xF, true);      // quad_perm [1,0,3,2]
  } else if constexpr (M == 2) {
    r = __builtin_amdgcn_mov_dpp(v, 0x4E, 0xF, 0xF, true);      // quad_perm [2,3,0,1]
  } else if constexpr (M == 4) {
    r = __builtin_amdgcn_ds_swizzle(v, 0x101F);                 // xor 4 (bitmask mode)
  } else if constexpr (M == 8) {
    r = __builtin_amdgcn_mov_dpp(v, 0x128, 0xF, 0xF, true);     // row_ror:8 == xor 8 in a row
  } else if constexpr (M == 16) {
    const auto p = __builtin_amdgcn_permlane16_swap((uint32_t)v, (uint32_t)v, false, false);
    r = (int)((__lane_id() & 16) ? p[0] : p[1]);
  } else {
    static_assert(M == 32, "xor_lane: unsupported mask");
    const auto p = __builtin_amdgcn_permlane32_swap((uint32_t)v, (uint32_t)v, false, false);
    r = (int)((__lane_id() & 32) ? p[0] : p[1]);
  }
  return __int_as_float(r);
}

// x + (x of lane ^ M) for the reductions: any pairing works once the lower
// levels are summed, so M = 4 and 8 use the DPP mirrors and 16, 32 add the
// two halves of a permlane swap (no lane select).
template <int M>
__device__ __forceinline__ float pair_sum(float x) {
  const int v = __float_as_int(x);
  if constexpr (M == 1 || M == 2) {
    return x + xor_lane<M>(x);
  } else if constexpr (M == 4) {
    return x + __int_as_float(__builtin_amdgcn_mov_dpp(v, 0x141, 0xF, 0xF, true));  // half mirror
  } else if constexpr (M == 8) {
    return x + __int_as_float(__builtin_amdgcn_mov_dpp(v, 0x140, 0xF, 0xF, true));  // row mirror
  } else if constexpr (M == 16) {
    const auto p = __builtin_amdgcn_permlane16_swap((uint32_t)v, (uint32_t)v, false, false);
    return __uint_as_float(p[0]) + __uint_as_float(p[1]);
  } else {
    static_assert(M == 32, "pair_sum: unsupported mask");
    const auto p = __builtin_amdgcn_permlane32_swap((uint32_t)v, (uint32_t)v, false, false);
    return __uint_as_float(p[0]) + __uint_as_float(p[1]);
  }
}
template <int M>
__device__ __forceinline__ float pair_max(float x) {
  const int v = __float_as_int(x);
  if constexpr (M == 1 || M == 2) {
    return fmaxf(x, xor_lane<M>(x));
  } else if constexpr (M == 4) {
    return fmaxf(x, __int_as_float(__builtin_amdgcn_mov_dpp(v, 0x141, 0xF, 0xF, true)));
  } else if constexpr (M == 8) {
    return fmaxf(x, __int_as_float(__builtin_amdgcn_mov_dpp(v, 0x140, 0xF, 0xF, true)));
  } else if constexpr (M == 16) {
    const auto p = __builtin_amdgcn_permlane16_swap((uint32_t)v, (uint32_t)v, false, false);
    return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
  } else {
    static_assert(M == 32, "pair_max: unsupported mask");
    const auto p = __builtin_amdgcn_permlane32_swap((uint32_t)v, (uint32_t)v, false, false);
    return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
  }
}
template <int M>
__device__ __forceinline__ uint32_t pair_sum_u32(uint32_t v) {
  if constexpr (M == 1) {
    return v + (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, true);
  } else if constexpr (M == 2) {
    return v + (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, true);
  } else if constexpr (M == 4) {
    return v + (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x141, 0xF, 0xF, true);
  } else if constexpr (M == 8) {
    return v + (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x140, 0xF, 0xF, true);
  } else if constexpr (M == 16) {
    const auto p = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    return p[0] + p[1];
  } else {
    static_assert(M == 32, "pair_sum_u32: unsupported mask");
    const auto p = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return p[0] + p[1];
  }
}

// Walsh-Hadamard butterfly over one row of D = E*L elements held by L
// consecutive lanes (L in {1,2,4,8,16,32}), E consecutive elements per lane:
// element index = (lane % L) * E + i.  Unnormalised (entries +-1); the caller
// scales by 1/sqrt(D).  All lanes of the wavefront must execute this.
template <int E, int L>
__device__ __forceinline__ void hadamard_row(float (&v)[E], int lane) {
#pragma unroll
  for (int h = 1; h < E; h <<= 1) {
#pragma unroll
    for (int i = 0; i < E; ++i) {
      if ((i & h) == 0) {
        float a = v[i], b = v[i + h];
        v[i] = a + b;
        v[i + h] = a - b;
      }
    }
  }
#define KVQ_XSTAGE(MASK)                                              \
  if constexpr (L > (MASK)) {                                         \
    const float sg = (lane & (MASK)) ? -1.0f : 1.0f;                  \
    _Pragma("unroll") for (int i = 0; i < E; ++i) {                   \
      float p = xor_lane<(MASK)>(v[i]);                               \
      v[i] = __builtin_fmaf(v[i], sg, p);                             \
    }                                                                 \
  }
  KVQ_XSTAGE(1)
  KVQ_XSTAGE(2)
  KVQ_XSTAGE(4)
  KVQ_XSTAGE(8)
  KVQ_XSTAGE(16)
#undef KVQ_XSTAGE
}

// The same butterfly in float64 (each exchange moves the two 32-bit halves).
// With the non-packed float32 rate for float64 adds on gfx950, it costs what
// the float32 butterfly costs twice; it is exact for 2-byte inputs (their
// 8- or 11-bit significands summed over at most 256 terms fit 53 bits).
template <int M>
__device__ __forceinline__ double xor_lane_f64(double x) {
  const uint64_t u = __double_as_longlong(x);
  const float lo = xor_lane<M>(__uint_as_float((uint32_t)u));
  const float hi = xor_lane<M>(__uint_as_float((uint32_t)(u >> 32)));
  return __longlong_as_double((long long)(((uint64_t)__float_as_uint(hi) << 32) |
                                          __float_as_uint(lo)));
}
template <int E, int L>
__device__ __forceinline__ void hadamard_row_f64(double (&v)[E], int lane) {
#pragma unroll
  for (int h = 1; h < E; h <<= 1) {
#pragma unroll
    for (int i = 0; i < E; ++i) {
      if ((i & h) == 0) {
        const double a = v[i], b = v[i + h];
        v[i] = a + b;
        v[i + h] = a - b;
      }
    }
  }
#define KVQ_XSTAGE_D(MASK)                                            \
  if constexpr (L > (MASK)) {                                         \
    const bool up = (lane & (MASK)) != 0;                             \
    _Pragma("unroll") for (int i = 0; i < E; ++i) {                   \
      const double p = xor_lane_f64<(MASK)>(v[i]);                    \
      v[i] = up ? p - v[i] : v[i] + p;                                \
    }                                                                 \
  }
  KVQ_XSTAGE_D(1)
  KVQ_XSTAGE_D(2)
  KVQ_XSTAGE_D(4)
  KVQ_XSTAGE_D(8)
  KVQ_XSTAGE_D(16)
#undef KVQ_XSTAGE_D
}

// Sum over the L consecutive lanes of a row (L a power of two <= 32); every
// lane of the row receives the sum.  All lanes of the wavefront execute this.
template <int L>
__device__ __forceinline__ float row_sum(float x) {
  if constexpr (L > 1) x = pair_sum<1>(x);
  if constexpr (L > 2) x = pair_sum<2>(x);
  if constexpr (L > 4) x = pair_sum<4>(x);
  if constexpr (L > 8) x = pair_sum<8>(x);
  if constexpr (L > 16) x = pair_sum<16>(x);
  return x;
}

// Wavefront reductions (all 64 lanes participate), VALU only: DPP within
// rows, permlane swaps across them.
__device__ __forceinline__ float wave_max(float x) {
  x = pair_max<1>(x);
  x = pair_max<2>(x);
  x = pair_max<4>(x);
  x = pair_max<8>(x);
  x = pair_max<16>(x);
  return pair_max<32>(x);
}
__device__ __forceinline__ float wave_sum(float x) {
  x = pair_sum<1>(x);
  x = pair_sum<2>(x);
  x = pair_sum<4>(x);
  x = pair_sum<8>(x);
  x = pair_sum<16>(x);
  return pair_sum<32>(x);
}
__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t v) {
  v = pair_sum_u32<1>(v);
  v = pair_sum_u32<2>(v);
  v = pair_sum_u32<4>(v);
  v = pair_sum_u32<8>(v);
  v = pair_sum_u32<16>(v);
  return pair_sum_u32<32>(v);
}

__device__ __forceinline__ constexpr double rsqrt_pow2_f64(int d) {
  // 1/sqrt(d) rounded to float64, d in {64, 128, 256}.
  return d == 64 ? 0.125 : d == 128 ? 0.08838834764831843 : 0.0625;
}

// ceil(log2 x) for a finite float x >= 1 (exact: from the exponent field,
// plus one when any mantissa bit is set).
__device__ __forceinline__ int ceil_log2_f(float x) {
  const uint32_t u = __float_as_uint(x);
  const int e = (int)((u >> 23) & 255u) - 127;
  return e + ((u & 0x7fffffu) != 0u ? 1 : 0);
}

__device__ __forceinline__ constexpr float rsqrt_pow2(int d) {
  // 1/sqrt(d) for d in {1,...,256} powers of two, exact to float rounding.
  return d == 64 ? 0.125f
       : d == 128 ? 0.08838834764831845f
       : d == 256 ? 0.0625f
       : d == 32 ? 0.17677669529663688f
       : d == 16 ? 0.25f
       : d == 8 ? 0.3535533905932738f
       : d == 4 ? 0.5f
       : d == 2 ? 0.7071067811865476f : 1.0f;
}

}  // namespace kvq
