// K1 -- orthonormal Walsh-Hadamard rotation of rows, y = H_D x.
//
// Rotation step of the encode path ("ZeroKV-Neo 4.0.0", Architecture: FWHT
// energy spreading before quantisation; "VeloxQuant-MLX 0.5.1", VecInfer:
// Walsh-Hadamard rotation).  HBM-bound: each row is read once (2 or 4 bytes
// per element) and written once as float32.
//
// Layout: one row is held by L = D/8 consecutive lanes, 8 elements per lane,
// so a wavefront covers 64/L rows and each lane moves one 16-byte (bf16/f16)
// or 32-byte (f32) contiguous piece: fully coalesced.  Butterflies on the 3
// in-lane bits are register adds; the cross-lane bits use DPP / ds_swizzle.
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
  const int col = lane % L;        // 8-element piece within the row
  const char* xb = reinterpret_cast<const char*>(x);
  for (int64_t base = ((int64_t)blockIdx.x * (blockDim.x >> 6) + wave) * ROWS_PER_WAVE;
       base < n_rows; base += waves_total * ROWS_PER_WAVE) {
    const int64_t row = base + sub;
    const bool live = row < n_rows;
    const int64_t r_ld = live ? row : (n_rows - 1);  // keep every lane in the exchanges
    float v[8];
    load8<XT>(xb + (r_ld * D + (int64_t)col * 8) * ESZ, v);
    hadamard_row<8, L>(v, lane);
    constexpr float sc = rsqrt_pow2(D);
    if (live) {
      float4* o = reinterpret_cast<float4*>(y + row * D + col * 8);
      o[0] = make_float4(v[0] * sc, v[1] * sc, v[2] * sc, v[3] * sc);
      o[1] = make_float4(v[4] * sc, v[5] * sc, v[6] * sc, v[7] * sc);
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
