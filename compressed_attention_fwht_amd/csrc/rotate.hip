// K1 -- orthonormal Walsh-Hadamard rotation of rows, y = H_D x.
//
// Rotation step of the encode path ("ZeroKV-Neo 4.0.0", Architecture: FWHT
// energy spreading before quantisation; "VeloxQuant-MLX 0.5.1", VecInfer:
// Walsh-Hadamard rotation).  HBM-bound: each row is read once (2 or 4 bytes
// per element) and written once as float32.
//
// Layout: one row is held by L = D/8 consecutive lanes, 8 elements per lane:
// lane c holds elements [4c, 4c+4) and [D/2 + 4c, D/2 + 4c + 4), so each of
// its two loads and two 16-byte stores lands next to its neighbours'.  That
// layout permutes the bits of the element index (the top bit becomes the
// in-lane bit 2); the Walsh-Hadamard matrix is unchanged by the same bit
// permutation of rows and columns, so the butterfly over (lane, element)
// computes the transform.  Butterflies on the 3 in-lane bits are register
// adds; the cross-lane bits use DPP / ds_swizzle.
#include "kvq_internal.h"

namespace kvq {

template <int XT, int D>
__global__ __launch_bounds__(256) void rotate_kernel(const void* x,
                                                     float* y, int64_t n_rows) {  // x may alias y (f32 in place)
  constexpr int L = D / 8;
  constexpr int ROWS_PER_WAVE = 64 / L;
  constexpr int ESZ = XT == 0 ? 4 : 2;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t waves_total = (int64_t)gridDim.x * (blockDim.x >> 6);
  const int sub = lane / L;        // row within the wave's group
  const int col = lane % L;        // the lane's place within the row
  const char* xb = reinterpret_cast<const char*>(x);
  for (int64_t base = ((int64_t)blockIdx.x * (blockDim.x >> 6) + wave) * ROWS_PER_WAVE;
       base < n_rows; base += waves_total * ROWS_PER_WAVE) {
    const int64_t row = base + sub;
    const bool live = row < n_rows;
    const int64_t r_ld = live ? row : (n_rows - 1);  // keep every lane in the exchanges
    const int da = 4 * col, db = D / 2 + 4 * col;
    float v[8];
    load4<XT>(xb + (r_ld * D + da) * ESZ, v, 0);
    load4<XT>(xb + (r_ld * D + db) * ESZ, v, 4);
    hadamard_row<8, L>(v, lane);
    constexpr float sc = rsqrt_pow2(D);
    if (live) {
      *reinterpret_cast<float4*>(y + row * D + da) = make_float4(v[0] * sc, v[1] * sc, v[2] * sc, v[3] * sc);
      *reinterpret_cast<float4*>(y + row * D + db) = make_float4(v[4] * sc, v[5] * sc, v[6] * sc, v[7] * sc);
    }
  }
}

template <int XT, int D>
static hipError_t launch_rotate_t(const void* x, float* y, int64_t n_rows, hipStream_t s) {
  constexpr int ROWS_PER_BLOCK = 4 * (64 / (D / 8));
  int64_t blocks = (n_rows + ROWS_PER_BLOCK - 1) / ROWS_PER_BLOCK;
  if (blocks > 65536) blocks = 65536;
  rotate_kernel<XT, D><<<dim3((unsigned)blocks), dim3(256), 0, s>>>(x, y, n_rows);
  return hipGetLastError();
}

hipError_t launch_rotate(const void* x, int xt, float* y, int64_t n_rows, int dim, hipStream_t s) {
  if (n_rows == 0) return hipSuccess;
#define KVQ_ROT(XT)                                                          \
  if (dim == 64) return launch_rotate_t<XT, 64>(x, y, n_rows, s);            \
  if (dim == 128) return launch_rotate_t<XT, 128>(x, y, n_rows, s);          \
  return launch_rotate_t<XT, 256>(x, y, n_rows, s);
  if (xt == 0) { KVQ_ROT(0) }
  if (xt == 1) { KVQ_ROT(1) }
  KVQ_ROT(2)
#undef KVQ_ROT
}

}  // namespace kvq
