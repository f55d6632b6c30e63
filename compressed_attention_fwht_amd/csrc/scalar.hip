// Scalar residual variant: two-pass scalar quantisation of the rotated vector
// with sub-byte index packing.
//
// "VeloxQuant-MLX 0.5.1": Architecture, TurboQuantRVQ pipeline -- rotate,
// stage-1 Gaussian Lloyd-Max scalar quantiser, residual, stage-2 Laplacian
// Lloyd-Max, the indices only, decode by summing the two levels and
// unrotating; throughput journey -- the index as a sum over decision
// boundaries instead of an argmin (same indices); module table --
// dsa.bit_pack sub-byte packing.
//
// Codes: a vector's row is [stage-1 bytes][stage-2 bytes], D*b/8 bytes each;
// a stage is one bit string, least significant bit first: bit t of element i
// is bit i*b + t of the stage's bytes.  For b in {1, 2, 4} element i sits in
// bits [(i mod k)*b, ...) of byte i / k (k = 8/b), so a byte of stage s is a
// code of the product codebook whose entry c lists levels_s[(c >> j*b) &
// (2^b - 1)] for j < k -- scalar_product_cb_kernel writes it, and the
// decode-attention kernels read packed scalar codes as ordinary product codes
// (G = D*b/8 groups of k dims, C = 256).  For b = 3 elements straddle bytes:
// encode and reconstruction only.
//
// Encode: 32 consecutive elements per lane (D/32 lanes per row), so a lane's
// indices fill b whole 32-bit words per stage; reconstruction: D/8 lanes per
// row.  In principle HBM-bound: 2 (or 4) bytes in and b/4 bytes out per
// element.
#include <math.h>

#include "kvq_internal.h"

namespace kvq {

// -------------------------------------------------------------- Lloyd-Max
// Moments of a unit-variance density over [a, b] (a < b, either may be
// infinite): mass, first and second moments, in closed form.
namespace {
struct Moments {
  double m0, m1, m2;
};

constexpr double kPi = 3.14159265358979323846;
inline double phi(double t) { return isinf(t) ? 0.0 : exp(-0.5 * t * t) / sqrt(2.0 * kPi); }
inline double Phi(double t) { return 0.5 * erfc(-t / sqrt(2.0)); }

Moments gauss_moments(double a, double b) {
  // int phi = Phi(b) - Phi(a); int t phi = phi(a) - phi(b);
  // int t^2 phi = Phi(b) - Phi(a) - (b phi(b) - a phi(a))
  const double ta = isinf(a) ? 0.0 : a * phi(a), tb = isinf(b) ? 0.0 : b * phi(b);
  const double m0 = Phi(b) - Phi(a);
  return {m0, phi(a) - phi(b), m0 - (tb - ta)};
}

// Laplace with scale beta = 1/sqrt(2) (unit variance), on [a, b] with a >= 0:
// int_a^b e^(-x/beta) / (2 beta) x^n dx through the antiderivatives.
Moments laplace_pos(double a, double b) {
  const double be = 1.0 / sqrt(2.0);
  auto F = [&](double x, int n) -> double {          // value of -0.5 e^(-x/be) P_n(x)
    if (isinf(x)) return 0.0;
    const double e = exp(-x / be);
    if (n == 0) return -0.5 * e;
    if (n == 1) return -0.5 * e * (x + be);
    return -0.5 * e * (x * x + 2.0 * be * x + 2.0 * be * be);
  };
  return {F(b, 0) - F(a, 0), F(b, 1) - F(a, 1), F(b, 2) - F(a, 2)};
}

Moments laplace_moments(double a, double b) {
  if (a >= 0.0) return laplace_pos(a, b);
  if (b <= 0.0) {                                     // mirror: x -> -x
    const Moments m = laplace_pos(-b, -a);
    return {m.m0, -m.m1, m.m2};
  }
  const Moments l = laplace_pos(0.0, -a), r = laplace_pos(0.0, b);
  return {l.m0 + r.m0, r.m1 - l.m1, l.m2 + r.m2};
}
}  // namespace

int lloyd_max(int kind, int bits, double* levels, double* distortion) {
  const int n = 1 << bits;
  auto mom = [&](double a, double b) {
    return kind == 0 ? gauss_moments(a, b) : laplace_moments(a, b);
  };
  for (int k = 0; k < n; ++k) levels[k] = n > 1 ? -2.0 + 4.0 * k / (n - 1) : 0.0;
  double edges[17];
  for (int it = 0; it < 100000; ++it) {
    edges[0] = -INFINITY;
    edges[n] = INFINITY;
    for (int k = 1; k < n; ++k) edges[k] = 0.5 * (levels[k - 1] + levels[k]);
    double moved = 0.0;
    for (int k = 0; k < n; ++k) {
      const Moments m = mom(edges[k], edges[k + 1]);
      const double c = m.m1 / m.m0;
      moved = fmax(moved, fabs(c - levels[k]));
      levels[k] = c;
    }
    if (moved < 1e-15) break;
  }
  if (distortion) {
    edges[0] = -INFINITY;
    edges[n] = INFINITY;
    for (int k = 1; k < n; ++k) edges[k] = 0.5 * (levels[k - 1] + levels[k]);
    double d = 0.0;
    for (int k = 0; k < n; ++k) {                     // int (t - c)^2 = m2 - 2 c m1 + c^2 m0
      const Moments m = mom(edges[k], edges[k + 1]);
      d += m.m2 - 2.0 * levels[k] * m.m1 + levels[k] * levels[k] * m.m0;
    }
    *distortion = d;
  }
  return 0;
}

// ---------------------------------------------------------------- kernels
// Levels of the block's book staged in LDS with the decision thresholds
// (midpoints of neighbouring levels, float32).
template <int B>
__device__ __forceinline__ void stage_levels(const float* __restrict__ levels, int64_t book,
                                             float (&lv)[2][1 << B], float (&th)[2][1 << B]) {
  constexpr int NL = 1 << B;
  const int tid = threadIdx.x;
  if (tid < 2 * NL) lv[tid / NL][tid % NL] = levels[book * 2 * NL + tid];
  __syncthreads();
  if (tid < 2 * NL && tid % NL < NL - 1)
    th[tid / NL][tid % NL] = 0.5f * (lv[tid / NL][tid % NL] + lv[tid / NL][tid % NL + 1]);
  __syncthreads();
}

// Number of thresholds strictly below v: the test v > t is the sign bit of
// t - v (t - v is +0 when they are equal, so equality counts as "not above",
// like the strict comparison) -- integer work, no comparison mask.
template <int B>
__device__ __forceinline__ uint32_t bsum(float v, const float (&th)[1 << B]) {
  uint32_t z = 0u;
#pragma unroll
  for (int k = 0; k < (1 << B) - 1; ++k) z += __float_as_uint(th[k] - v) >> 31;
  return z;
}

// rows per lane per pass: their loads are all issued before any of them is
// used, so each wave keeps SC_U loads in flight (a streaming kernel is bound by
// the bytes in flight, not by its arithmetic)
constexpr int SC_U = 4;

// Encode layout: SE_E consecutive elements per lane (L = D/SE_E lanes per
// row, 2, 4 or 8), so the 128-point butterfly has five in-register stages
// and two cross-lane ones (each cross-lane stage moves both 32-bit halves of
// every float64 element and selects around them, the costly part), and a
// lane's indices fill SE_E*b/32 whole words per stage.  SE_U rows per lane
// and pass.
constexpr int SE_E = 32;
constexpr int SE_U = 1;

// grid (row blocks, n_books), 256 threads; grid-stride over the book's rows.
template <int D, int XT, int B>
__global__ __launch_bounds__(256) void scalar_encode_kernel(
    const void* __restrict__ x, const float* __restrict__ levels, uint8_t* __restrict__ codes,
    int64_t n_seq, int64_t seq_stride, int64_t n_rows, int pre_rotated, uint64_t dm, int dsh) {
  constexpr int E = SE_E;
  constexpr int L = D / E;
  constexpr int RPB = 256 / L;                          // rows per block and unroll step
  constexpr int ESZ = XT == 0 ? 4 : 2;
  constexpr int SB = D * B / 8;                         // bytes per stage
  constexpr int NW = E * B / 32;                        // code words per lane and stage
  __shared__ float lv[2][1 << B], th[2][1 << B];
  const int64_t book = blockIdx.y;
  stage_levels<B>(levels, book, lv, th);
  const int tid = threadIdx.x, lane = tid & 63;
  const int col = tid % L, rsub = tid / L;
  const int64_t n = n_seq * n_rows;
  float t0[1 << B], t1[1 << B];                         // the thresholds, in registers
#pragma unroll
  for (int k = 0; k < (1 << B); ++k) {
    t0[k] = th[0][k];
    t1[k] = th[1][k];
  }
  for (int64_t base = (int64_t)blockIdx.x * RPB * SE_U; base < n;
       base += (int64_t)gridDim.x * RPB * SE_U) {
    // The rotation runs in float64 (exact for 2-byte inputs), each element is
    // rounded once to float32 for the stage-1 threshold tests, and the
    // stage-2 residual y - level is taken in float64 before its own rounding:
    // a test then errs only when the element lies within about 1e-7 of its
    // magnitude from a threshold, far inside the 1e-4 near-tie rule for
    // every level spacing of b <= 4.  All SE_U rows' loads go out first.
    double yd[SE_U][E];
#pragma unroll
    for (int u = 0; u < SE_U; ++u) {
      const int64_t v = base + u * RPB + rsub;
      const int64_t vl = v < n ? v : n - 1;             // every lane joins the butterfly
      // vl / n_rows by multiply and shift when both fit 31 bits (dsh != 0)
      const int64_t seq = dsh ? (int64_t)(((uint64_t)vl * dm) >> dsh) : vl / n_rows;
      const int64_t row = vl - seq * n_rows;
      const char* src = reinterpret_cast<const char*>(x) +
                        (((book * n_seq + seq) * seq_stride + row) * D + col * E) * ESZ;
#pragma unroll
      for (int c = 0; c < E / 8; ++c) {
        float f[8];
        load8<XT>(src + c * 8 * ESZ, f);
#pragma unroll
        for (int e = 0; e < 8; ++e) yd[u][8 * c + e] = (double)f[e];
      }
    }
    uint32_t p1[SE_U][NW], p2[SE_U][NW];
#pragma unroll
    for (int u = 0; u < SE_U; ++u) {
      if (!pre_rotated) hadamard_row_f64<E, L>(yd[u], lane);
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        p1[u][w] = 0u;
        p2[u][w] = 0u;
      }
#pragma unroll
      for (int e = 0; e < E; ++e) {
        double y = yd[u][e];
        if (!pre_rotated) y *= rsqrt_pow2_f64(D);
        const uint32_t z1 = bsum<B>((float)y, t0);
        const uint32_t z2 = bsum<B>((float)(y - (double)lv[0][z1]), t1);
        // bits [e*B, e*B + B) of the lane's stage words (a 3-bit index may
        // straddle two words)
        const int bit = e * B, w = bit >> 5, sh = bit & 31;
        p1[u][w] |= z1 << sh;
        p2[u][w] |= z2 << sh;
        if (sh + B > 32) {
          p1[u][w + 1] |= z1 >> (32 - sh);
          p2[u][w + 1] |= z2 >> (32 - sh);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < SE_U; ++u) {
      const int64_t v = base + u * RPB + rsub;
      if (v < n) {
        uint8_t* rowp = codes + (book * n + v) * (2 * SB) + col * (E * B / 8);
        uint32_t* a = reinterpret_cast<uint32_t*>(rowp);      // 4-byte aligned: E*B/8 = 4*NW
        uint32_t* b = reinterpret_cast<uint32_t*>(rowp + SB);
        if constexpr (NW == 2) {
          *reinterpret_cast<uint2*>(a) = make_uint2(p1[u][0], p1[u][1]);
          *reinterpret_cast<uint2*>(b) = make_uint2(p2[u][0], p2[u][1]);
        } else if constexpr (NW == 4) {
          *reinterpret_cast<uint4*>(a) = make_uint4(p1[u][0], p1[u][1], p1[u][2], p1[u][3]);
          *reinterpret_cast<uint4*>(b) = make_uint4(p2[u][0], p2[u][1], p2[u][2], p2[u][3]);
        } else {
#pragma unroll
          for (int w = 0; w < NW; ++w) {
            a[w] = p1[u][w];
            b[w] = p2[u][w];
          }
        }
      }
    }
  }
}

// grid (row blocks, n_books); out = levels1[z1] + levels2[z2] (one float32
// rounding of the sum), then H_D when unrotate.  Lane c of a row holds dims
// [4c, 4c+4) and [D/2 + 4c, D/2 + 4c + 4): a permutation of the dim index
// bits, under which the same butterfly computes the transform, and which puts
// each 16-byte store next to its neighbours'.  The 4 indices of a half sit
// in 4*B consecutive bits of the packed row.
template <int B>
__device__ __forceinline__ uint32_t scalar_bits4(const uint8_t* __restrict__ rowp, int d0) {
  const int bit = d0 * B;                               // 4*B bits from here (d0 % 4 == 0)
  if constexpr (B == 1) return (uint32_t)(rowp[bit >> 3] >> (bit & 7)) & 15u;
  else if constexpr (B == 2) return rowp[bit >> 3];
  else if constexpr (B == 3) {                          // 12 bits from bit 0 or 4 of a byte
    const uint32_t two = (uint32_t)rowp[bit >> 3] | ((uint32_t)rowp[(bit >> 3) + 1] << 8);
    return (two >> (bit & 7)) & 0xfffu;
  } else return *reinterpret_cast<const uint16_t*>(rowp + (bit >> 3));
}

template <int D, int B>
__global__ __launch_bounds__(256) void scalar_reconstruct_kernel(
    const uint8_t* __restrict__ codes, const float* __restrict__ levels, float* __restrict__ out,
    int64_t n, int unrotate) {
  constexpr int L = D / 8;
  constexpr int RPB = 256 / L;
  constexpr int SB = D * B / 8;
  constexpr uint32_t MASK = (1u << B) - 1u;
  __shared__ float lv[2][1 << B], th[2][1 << B];
  const int64_t book = blockIdx.y;
  stage_levels<B>(levels, book, lv, th);
  const int tid = threadIdx.x, lane = tid & 63;
  const int col = tid % L, rsub = tid / L;
  const int da = 4 * col, db = D / 2 + 4 * col;
  for (int64_t base = (int64_t)blockIdx.x * RPB * SC_U; base < n;
       base += (int64_t)gridDim.x * RPB * SC_U) {
    uint32_t p1a[SC_U], p1b[SC_U], p2a[SC_U], p2b[SC_U];
#pragma unroll
    for (int u = 0; u < SC_U; ++u) {
      const int64_t v = base + u * RPB + rsub;
      const int64_t vl = v < n ? v : n - 1;
      const uint8_t* rowp = codes + (book * n + vl) * (2 * SB);
      p1a[u] = scalar_bits4<B>(rowp, da);
      p1b[u] = scalar_bits4<B>(rowp, db);
      p2a[u] = scalar_bits4<B>(rowp + SB, da);
      p2b[u] = scalar_bits4<B>(rowp + SB, db);
    }
#pragma unroll
    for (int u = 0; u < SC_U; ++u) {
      const int64_t v = base + u * RPB + rsub;
      float y[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        y[e] = lv[0][(p1a[u] >> (e * B)) & MASK] + lv[1][(p2a[u] >> (e * B)) & MASK];
        y[4 + e] = lv[0][(p1b[u] >> (e * B)) & MASK] + lv[1][(p2b[u] >> (e * B)) & MASK];
      }
      if (unrotate) {
        hadamard_row<8, L>(y, lane);
        constexpr float sc = rsqrt_pow2(D);
#pragma unroll
        for (int e = 0; e < 8; ++e) y[e] *= sc;
      }
      if (v < n) {
        float* o = out + (book * n + v) * D;
        *reinterpret_cast<float4*>(o + da) = make_float4(y[0], y[1], y[2], y[3]);
        *reinterpret_cast<float4*>(o + db) = make_float4(y[4], y[5], y[6], y[7]);
      }
    }
  }
}

// cb[s][g][c][j] = levels_s[(c >> j*B) & MASK], j < 8/B, the same for every g.
template <int B>
__global__ __launch_bounds__(256) void scalar_product_cb_kernel(const float* __restrict__ levels,
                                                                float* __restrict__ cb, int G) {
  constexpr int K = 8 / B;
  constexpr uint32_t MASK = (1u << B) - 1u;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;    // (s, g, c)
  if (i >= (int64_t)2 * G * 256) return;
  const int c = (int)(i % 256);
  const int s = (int)(i / ((int64_t)G * 256));
  float* dst = cb + i * K;
#pragma unroll
  for (int j = 0; j < K; ++j) dst[j] = levels[s * (1 << B) + ((c >> (j * B)) & MASK)];
}

// ---------------------------------------------------------------- launchers
static unsigned row_grid(int64_t n, int D, int per_lane = 8, int rows_per_lane = SC_U) {
  const int64_t rpb = 256 / (D / per_lane) * rows_per_lane;
  int64_t b = (n + rpb - 1) / rpb;
  if (b > 4096) b = 4096;
  return (unsigned)(b > 0 ? b : 1);
}

hipError_t launch_scalar_encode(const void* x, int xt, int D, int bits, int64_t n_books,
                                int64_t n_seq, int64_t seq_stride, int64_t n_rows,
                                const float* levels, uint8_t* codes, int pre_rotated,
                                hipStream_t st) {
  const int64_t n = n_seq * n_rows;
  if (n == 0 || n_books == 0) return hipSuccess;
  const dim3 grid(row_grid(n, D, SE_E, SE_U), (unsigned)n_books);
  // q = floor(v / n_rows) = (v * m) >> (31 + l) for every v < 2^31, with
  // l = ceil(log2 n_rows) and m = ceil(2^(31+l) / n_rows) (Granlund and
  // Montgomery, "Division by invariant integers using multiplication", 1994)
  uint64_t dm = 0;
  int dsh = 0;
  if (n < ((int64_t)1 << 31)) {
    int l = 0;
    while (((int64_t)1 << l) < n_rows) ++l;
    dm = (((uint64_t)1 << (31 + l)) + (uint64_t)n_rows - 1) / (uint64_t)n_rows;
    dsh = 31 + l;
  }
#define KVQ_SE(DD, XX, BB)                                                                 \
  if (D == DD && xt == XX && bits == BB) {                                                \
    scalar_encode_kernel<DD, XX, BB><<<grid, dim3(256), 0, st>>>(x, levels, codes, n_seq,  \
                                                                 seq_stride, n_rows,       \
                                                                 pre_rotated, dm, dsh);    \
    return hipGetLastError();                                                              \
  }
#define KVQ_SE_X(DD, XX)                                                                  \
  KVQ_SE(DD, XX, 1) KVQ_SE(DD, XX, 2) KVQ_SE(DD, XX, 3) KVQ_SE(DD, XX, 4)
#define KVQ_SE_D(DD) KVQ_SE_X(DD, 0) KVQ_SE_X(DD, 1) KVQ_SE_X(DD, 2)
  KVQ_SE_D(64) KVQ_SE_D(128) KVQ_SE_D(256)
#undef KVQ_SE_D
#undef KVQ_SE_X
#undef KVQ_SE
  return hipErrorInvalidValue;
}

hipError_t launch_scalar_reconstruct(const uint8_t* codes, int D, int bits, int64_t n_books,
                                     int64_t n, const float* levels, float* out, int unrotate,
                                     hipStream_t st) {
  if (n == 0 || n_books == 0) return hipSuccess;
  const dim3 grid(row_grid(n, D), (unsigned)n_books);
#define KVQ_SR(DD, BB)                                                                     \
  if (D == DD && bits == BB) {                                                             \
    scalar_reconstruct_kernel<DD, BB><<<grid, dim3(256), 0, st>>>(codes, levels, out, n,    \
                                                                  unrotate);               \
    return hipGetLastError();                                                              \
  }
  KVQ_SR(64, 1) KVQ_SR(64, 2) KVQ_SR(64, 3) KVQ_SR(64, 4) KVQ_SR(128, 1) KVQ_SR(128, 2)
  KVQ_SR(128, 3) KVQ_SR(128, 4) KVQ_SR(256, 1) KVQ_SR(256, 2) KVQ_SR(256, 3) KVQ_SR(256, 4)
#undef KVQ_SR
  return hipErrorInvalidValue;
}

hipError_t launch_scalar_product_cb(const float* levels, int D, int bits, float* cb,
                                    hipStream_t st) {
  const int G = D * bits / 8;
  const unsigned blocks = (unsigned)((2 * G * 256 + 255) / 256);
  if (bits == 1) scalar_product_cb_kernel<1><<<blocks, 256, 0, st>>>(levels, cb, G);
  else if (bits == 2) scalar_product_cb_kernel<2><<<blocks, 256, 0, st>>>(levels, cb, G);
  else scalar_product_cb_kernel<4><<<blocks, 256, 0, st>>>(levels, cb, G);
  return hipGetLastError();
}

}  // namespace kvq
